/*
 * moe.h -- C ABI of the MI355X latent sparse mixture-of-experts layer.
 *
 * One forward pass of the layer
 *     y   = P_up( sum_{j<k} w_j * N( E_{idx_j}( P_down u ) ) )
 *     out = h + g * y          (or out = y)
 * where u is the branch input (x, or an RMS norm of x), the gate
 * (idx, w) = Softmax(KeepTopK(u W_r^T, k)), E_e is expert e and N the
 * per-expert output norm.  Sources, cited by page title and section:
 *   - bobbyburns.tech, "816 billion parameters, and only 42 billion show up
 *     for each token", section "The math": "Setup" (y = sum_i G(x)_i E_i(x),
 *     experts with G_i = 0 are never evaluated) and "The gate"
 *     (G = Softmax(KeepTopK(H, k)), noise-free at inference);
 *   - flozi.net, "Muse Spark Open: Norm-Preserving Gates Are Not a Norm
 *     Guarantee": "Two normalization orders implement different functions"
 *     (R_eps, C_gamma, I_gamma with gain 1+gamma), "Latent experts:
 *     normalization happens before the weighted sum" (router on the
 *     full-width input, 8192 -> 4096 latent projection, SwiGLU experts with
 *     packed gate/up [n, 2F, L] and down [n, L, F] weights, one shared norm
 *     gain applied to every expert output before its routing weight) and
 *     "What this means for serving and kernel work" (FP32 router and gates,
 *     norms reduce in FP32 and return the input dtype);
 *   - archdb.vladsavinov.com, "Muse-Spark-Open-816B-A42B" fact sheet (SwiGLU,
 *     no GLU clamp, no FFN bias, no shared expert, routed scaling 1, latent
 *     width 4,096).
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE pointers (hipMalloc'd or from a
 *     framework allocator) owned by the caller; the library allocates
 *     nothing and is re-entrant; its only global state is the static
 *     scratch of moe_layer_forward_static and that array's per-device
 *     address, looked up once per device;
 *   - all matrices are row-major with the reduction dimension contiguous;
 *   - `stream` is a hipStream_t (NULL = default stream); work is enqueued
 *     asynchronously and no call synchronises with the host;
 *   - the descriptor is validated on the host before any launch; on error
 *     nothing is enqueued and a negative moe_status is returned;
 *   - MOE_ERR_HIP is the one status returned after launching began: a HIP
 *     launch or event call of the chain failed, the kernels before it may
 *     have been enqueued, and every output is undefined.  An error left
 *     pending by an earlier, unrelated HIP call on the calling thread is
 *     cleared when an entry point starts and is not reported by it;
 *   - inputs are assumed finite; there are no device-side checks.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,          /* malformed descriptor or NULL required pointer */
    MOE_ERR_UNSUPPORTED = -2,          /* well-formed, but a combination this build does not run */
    MOE_ERR_WORKSPACE_TOO_SMALL = -3,  /* workspace_bytes < moe_workspace_bytes(desc) */
    MOE_ERR_HIP = -4,                  /* a HIP launch or event call failed */
    MOE_ERR_STATIC_SCRATCH_TOO_SMALL = -5  /* moe_layer_forward_static: the batch needs more workspace
                                              than MOE_STATIC_SCRATCH_BYTES */
} moe_status;

enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_MXFP4 = 2, MOE_DT_F16 = 3 };
enum { MOE_NORM_NONE = 0, MOE_NORM_CENTERED = 1, MOE_NORM_INPUT_SCALED = 2 };
enum { MOE_EXPERT_RELU2 = 0, MOE_EXPERT_SWIGLU3 = 1 };
enum { MOE_RES_NONE = 0, MOE_RES_LINEAR = 1, MOE_RES_MUSE = 2 };
enum { MOE_ROUTER_SOFTMAX = 0, MOE_ROUTER_SIGMOID = 1 };
enum { MOE_AQ_NONE = 0, MOE_AQ_MXFP8 = 1 };

/* Number of timed stages; stage s is bracketed by stage_events[2s], [2s+1]. */
enum {
    MOE_STAGE_IN_NORM = 0, MOE_STAGE_ROUTER = 1, MOE_STAGE_TOPK = 2, MOE_STAGE_PERMUTE = 3,
    MOE_STAGE_DOWN = 4, MOE_STAGE_GEMM1 = 5, MOE_STAGE_GEMM2 = 6, MOE_STAGE_COMBINE = 7,
    MOE_STAGE_UP = 8, MOE_STAGE_RESGATE = 9, MOE_NUM_STAGES = 10
};

/*
 * Layer descriptor (host memory, read during the call only).
 *   T            tokens (rows of x); 0 is valid, enqueues nothing and
 *                accepts NULL tensor and workspace pointers.  The latent
 *                path takes batches with T * d_latent * 2 < 2^31 (the
 *                latent z below 2 GiB; split larger batches)
 *   d_model      width d of x and out
 *   d_latent     latent width L of the expert space; 0 = experts read u
 *   n_experts    n (1..256); top_k: k (1..min(n,16))
 *   d_ff         expert hidden width F
 *   expert_kind  MOE_EXPERT_SWIGLU3: E(z) = W2 (silu(Wg z) * (Wu z)),
 *                expert_w1 = [n][2F][L] (rows 0..F-1 gate, F..2F-1 up),
 *                expert_w2 = [n][L][F];
 *                MOE_EXPERT_RELU2: E(u) = W2 relu(W1 u), expert_w1 =
 *                [n][F][d], expert_w2 = [n][d][F] (no latent)
 *   act_dtype    dtype of x: MOE_DT_BF16 or MOE_DT_F32
 *   router_dtype dtype of router_w [n][d]; logits are always fp32
 *   weight_dtype dtype of down_w, expert_w1, expert_w2, up_w:
 *                F32, BF16, MXFP4, or F16: expert_w1, expert_w2 and up_w
 *                stored as IEEE fp16 and down_w as bf16 (the fp16 GEMMs
 *                then read their weights without converting them; a bf16
 *                checkpoint converts with moe_convert_bf16_to_f16, which
 *                changes no value in [2^-17, 65504], so the layer's results
 *                equal those of the BF16 format; needs fp16 intermediates).
 *                An MXFP4 matrix [R][K] is one buffer:
 *                R*K/2 bytes of E2M1 codes (row-major, low nibble = even
 *                element) followed by R*K/32 E8M0 scale bytes ([R][K/32]),
 *                one per 32 consecutive elements along K (OCP MX v1.0);
 *                an expert tensor is the [n*rows][K] matrix.
 *   in_norm      norm of x before router and down-projection (u = x if NONE)
 *   expert_norm  norm of each expert output before its routing weight
 *                (gain gamma_expert, one vector shared by all experts)
 *   res_gate     residual update of the branch output b (b = y, or the
 *                output norm of y when out_norm is set) with the residual x:
 *                MOE_RES_NONE: out = b; MOE_RES_LINEAR: out = x + g * b;
 *                MOE_RES_MUSE: out = alpha * x + beta * b, coordinate-wise
 *                with w = g / res_tau, beta = sigmoid(w), alpha =
 *                sqrt(max(sigmoid(-w) * (1 + beta), res_floor)) (flozi.net
 *                "Muse Spark Open: Norm-Preserving Gates Are Not a Norm
 *                Guarantee", "Residual gates: derive the advertised
 *                intuition carefully"; g = gains->res_gate, fp32 math)
 *   bias_in_weights  softmax router: 0 = router_bias only changes which
 *                experts are selected (weights use the unbiased logits);
 *                1 = it also enters the softmax.  Must be 0 for sigmoid.
 *   eps_in, eps_expert  RMS epsilons: R(v) = v * (mean(v^2) + eps)^-1/2
 *   interm_dtype dtype of the activations the latent path stores between
 *                its GEMMs and feeds to MFMA: the latent z, the SwiGLU
 *                output and the weighted sum m (the normalised expert
 *                outputs S stay bf16, the input dtype of that norm).
 *                MOE_DT_F16 (also selected by 0): 3 more mantissa bits than
 *                bf16; bf16/MXFP4 weights are converted to fp16 in registers
 *                (exact for 2^-17 <= |w| < 65504); a z or SwiGLU value of
 *                magnitude >= 65504 becomes +-inf and poisons its outputs.
 *                MOE_DT_BF16: bf16 everywhere (no range limit beyond bf16).
 *                Ignored on the fp32 path.
 *   router_fn    MOE_ROUTER_SOFTMAX (0): Softmax(KeepTopK) of the logits;
 *                MOE_ROUTER_SIGMOID: s = sigmoid(logit * router_out_mult)
 *                in fp32, selection on s + router_bias, weights = the kept
 *                s / (their sum + 1e-15) * routed_scale (same page, "Latent
 *                experts: normalization happens before the weighted sum").
 *                router_out_mult and routed_scale are read only for sigmoid.
 *   latent_norm  MOE_NORM_CENTERED: z = C_pre(P_down u), the output-scaled
 *                RMS norm of the latent with gain gains->gamma_latent [L]
 *                and eps_latent, before the experts read it (same page and
 *                section); MOE_NORM_NONE: z = P_down u.  Latent path only.
 *   out_norm     norm of the branch output y = P_up m before the residual
 *                gate (same page, "The complete layer has two separately
 *                normalized residual updates"): MOE_NORM_INPUT_SCALED,
 *                CENTERED (gain gains->gamma_out [d], eps_out; the scaled
 *                vector (1 + gamma) y is stored as bf16) or NONE.  Latent
 *                path only.
 *   res_tau, res_floor  MOE_RES_MUSE temperature (> 0; the page's default
 *                is 0.3) and floor (>= 0; 1e-3 on the page)
 *   act_quant    MOE_AQ_NONE (0), or MOE_AQ_MXFP8: the two expert GEMMs read
 *                MXFP8 activations (OCP MX v1.0: E4M3 elements, one E8M0
 *                scale 2^X per 32 consecutive values along K, X =
 *                floor(log2 max|v|) - 8, round to nearest even, magnitudes
 *                past 448 clamped), quantized from the stored latent z and
 *                the stored SwiGLU output (interm_dtype); with MXFP4 weights
 *                they run on the scaled fp8 x fp4 MFMA.  The router, the
 *                projections, norms and combine keep their precision.
 *                Needs weight_dtype MOE_DT_MXFP4 (the quantized-activation
 *                path of a 4-bit checkpoint, hefu.hk "Welcome Muse Spark
 *                Open", "Mixture of Experts Architecture").
 */
typedef struct {
    int64_t T;
    int64_t d_model;
    int64_t d_latent;
    int64_t n_experts;
    int64_t top_k;
    int64_t d_ff;
    int32_t expert_kind;
    int32_t act_dtype;
    int32_t router_dtype;
    int32_t weight_dtype;
    int32_t in_norm;
    int32_t expert_norm;
    int32_t res_gate;
    int32_t bias_in_weights;
    float eps_in;
    float eps_expert;
    int32_t interm_dtype;
    int32_t router_fn;
    float router_out_mult;
    float routed_scale;
    int32_t latent_norm;
    float eps_latent;
    int32_t out_norm;
    float eps_out;
    float res_tau;
    float res_floor;
    int32_t act_quant;
} moe_desc;

/* FP32 parameter vectors (device pointers; NULL where the stage is off).
 *   router_bias  [n]  selection bias (may be NULL even when routing)
 *   gamma_in     [d]  input-norm gain (gain applied as 1 + gamma)
 *   gamma_expert [L]  per-expert output-norm gain, shared by all experts
 *   res_gate     [d]  residual gate vector g (required by LINEAR and MUSE)
 *   gamma_latent [L]  latent pre-norm gain
 *   gamma_out    [d]  branch output-norm gain
 * A NULL gain means gamma = 0 (a gain of 1). */
typedef struct {
    const float *router_bias;
    const float *gamma_in;
    const float *gamma_expert;
    const float *res_gate;
    const float *gamma_latent;
    const float *gamma_out;
} moe_gains;

/* Optional outputs for inspection (device pointers, each may be NULL).
 *   topk_idx [T][k] int32  selected experts, largest score first, ties to
 *                          the lower expert id
 *   topk_w   [T][k] fp32   their gate weights
 *   expert_counts [n], expert_offsets [n+1] int32  tokens per expert and
 *                          the exclusive prefix sum
 *   perm_tok, perm_slot [T*k] int32  the (token, slot) pairs sorted by
 *                          (expert, token)
 *   y        [T][d] fp32   branch output b entering the residual gate (after
 *                          the output norm when out_norm is set)
 *   pos      [T][k] int32  perm position of (t, j)
 *   Intermediates of the bf16 latent path (ignored on the fp32 path):
 *   z        [T][L]  bf16  down-projection output (after the latent pre-norm)
 *   act      [T*k][F] bf16 SwiGLU output, rows in perm order
 *   S        [T*k][L] bf16 bf16((1+gamma) * expert output), perm order
 *   ssq      [T*k][L/16] fp32  per-16-column sums of squares of S (of the
 *                          unrounded expert output for the centered norm)
 *   m        [T][L]  bf16  weighted sum of the normalised expert outputs
 *   stage_events  NULL or an array of 2*MOE_NUM_STAGES hipEvent_t created
 *                 by the caller; stage s records [2s] before and [2s+1]
 *                 after its kernels on `stream` (skipped stages record
 *                 nothing)
 *   logits   [T][n] fp32   the router logits the selection used (the K
 *                          slices of the router GEMM already added, in
 *                          slice order)
 *   u        [T][d] act_dtype  the branch input the router and the
 *                          down-projection read: x, or its input norm
 *   zq, actq (act_quant = MXFP8) the MXFP8 forms of z [T][L] and of the
 *                          SwiGLU output [T*k][F] (perm order), each one
 *                          buffer: E4M3 codes [rows][K], then E8M0 scales
 *                          [rows][K/32] */
typedef struct {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *expert_counts;
    int32_t *expert_offsets;
    int32_t *perm_tok;
    int32_t *perm_slot;
    float *y;
    int32_t *pos;
    void *z;
    void *act;
    void *S;
    float *ssq;
    void *m;
    void **stage_events;
    float *logits;
    void *u;
    void *zq;
    void *actq;
} moe_debug;

/* Human-readable text of a moe_status (static storage). */
const char *moe_error_string(int status);

/* Host-only check of a descriptor: MOE_OK, MOE_ERR_INVALID_ARG or
 * MOE_ERR_UNSUPPORTED.  Needs no GPU.  What it checks is the shape of the
 * layer y = sum_i G(x)_i E_i(x) with a top-k gate over n experts
 * (bobbyburns.tech "816 billion parameters, and only 42 billion show up
 * for each token", "The math": "Setup" and "The gate": 1 <= k <= n) and of
 * the latent SwiGLU experts with their norms and residual gate (flozi.net
 * "Muse Spark Open: Norm-Preserving Gates Are Not a Norm Guarantee",
 * "Latent experts: normalization happens before the weighted sum"), plus
 * the size limits stated with moe_desc. */
int moe_validate(const moe_desc *desc);

/* Device workspace bytes moe_layer_forward needs for this descriptor
 * (0 if the descriptor is invalid).  Host-only; needs no GPU.  It holds
 * the layer's intermediates between its stages (the sections cited for
 * moe_validate): the router logits, the kept experts and weights, the
 * permutation of the (token, slot) pairs, the latent z, the SwiGLU
 * outputs and normalised expert outputs of the k selected experts of
 * every token, and the weighted sum m. */
size_t moe_workspace_bytes(const moe_desc *desc);

/*
 * The layer forward pass.
 *   x          [T][d]   act_dtype
 *   router_w   [n][d]   router_dtype
 *   down_w     [L][d]   weight_dtype (NULL when d_latent == 0)
 *   expert_w1, expert_w2  see moe_desc.expert_kind
 *   up_w       [d][L]   weight_dtype (NULL when d_latent == 0)
 *   gains      host struct of device vectors (may be NULL if none needed)
 *   out        [T][d]   fp32
 *   workspace  device scratch of at least moe_workspace_bytes(desc) bytes,
 *              256-byte aligned; contents on entry are ignored
 *   dbg        optional inspection outputs (NULL for none)
 * Returns MOE_OK once everything is enqueued on `stream`.  Without dbg the
 * call enqueues kernels only (no allocation, memset, copy or wait), so it may
 * be captured into a HIP graph; the replays reuse the captured pointers and
 * the workspace, so calls that overlap on one workspace race.
 */
int moe_layer_forward(const moe_desc *desc, const void *x, const void *router_w, const void *down_w,
                      const void *expert_w1, const void *expert_w2, const void *up_w,
                      const moe_gains *gains, void *out, void *workspace, size_t workspace_bytes,
                      moe_debug *dbg, void *stream);

/*
 * moe_layer_forward without a caller workspace and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a static device array of MOE_STATIC_SCRATCH_BYTES inside the
 * library: each device the library runs on holds its own copy from the first
 * call on it until the process ends.  Arguments, outputs and results are
 * those of moe_layer_forward (the same kernels run); the current HIP device
 * must be the one `stream` belongs to.
 *   - returns MOE_ERR_STATIC_SCRATCH_TOO_SMALL, before any launch, when
 *     moe_workspace_bytes(desc) > MOE_STATIC_SCRATCH_BYTES (at the
 *     816B-A42B layer shape: batches of more than 389 tokens, or 324 with
 *     the branch output norm);
 *   - calls no hipMalloc, hipFree or other allocating routine; the first
 *     call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress) and caches its address;
 *   - the forward reads no workspace byte before writing it, so nothing is
 *     cleared between calls; the array keeps the last call's intermediates;
 *   - every call on one device shares that device's array: calls that
 *     overlap on one device (concurrent streams, or threads enqueueing
 *     before the previous call's kernels have finished on another stream)
 *     race.  Calls enqueued on one stream are ordered and safe.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_forward_static(const moe_desc *desc, const void *x, const void *router_w, const void *down_w,
                             const void *expert_w1, const void *expert_w2, const void *up_w,
                             const moe_gains *gains, void *out, moe_debug *dbg, void *stream);

/*
 * Router stage alone: fp32 logits l = u W_r^T, then desc->router_fn:
 * softmax: selection on s = l + bias (fp32), top-k by (s descending,
 * expert id ascending), softmax of the kept logits ("The gate",
 * Softmax(KeepTopK)); sigmoid: see moe_desc.router_fn.  u is [T][d] of
 * desc->act_dtype (the branch input: no input norm is applied here).
 *   topk_idx [T][k] int32, topk_w [T][k] fp32 (outputs)
 *   logits   [T][n] fp32 (optional output, may be NULL)
 *   workspace >= moe_router_workspace_bytes(desc), required when logits is
 *            NULL.  For a bf16 router on a batch of more than 128 tokens
 *            and n a multiple of 256 the logits GEMM is split into K slices
 *            whose fp32 partial sums the workspace holds and the selection
 *            adds in slice order (deterministic); given logits and no
 *            workspace it runs unsplit.
 */
size_t moe_router_workspace_bytes(const moe_desc *desc);
int moe_router_topk(const moe_desc *desc, const void *u, const void *router_w, const float *router_bias,
                    int32_t *topk_idx, float *topk_w, float *logits, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Permutation stage alone.  It realises the sparse evaluation of
 * bobbyburns.tech "816 billion parameters, and only 42 billion show up for
 * each token", "The math" -> "Setup": an expert whose gate value is 0 is
 * never evaluated, so the (token, slot) pairs are grouped by the expert
 * they selected and each expert runs on its own rows only.
 * From topk_idx [T][k] (values in [0, n)) writes
 *   counts [n], offsets [n+1]  tokens per expert, exclusive prefix sum
 *   perm_tok, perm_slot [T*k]  pairs sorted by (expert, token): within
 *                              expert e's segment [offsets[e], offsets[e+1])
 *                              the tokens ascend
 *   pos [T][k]                 inverse: perm position of (t, j)
 * Deterministic (no atomics decide an order).  T*k < 2^31.
 */
int moe_permute(int64_t T, int64_t k, int64_t n, const int32_t *topk_idx, int32_t *counts, int32_t *offsets,
                int32_t *perm_tok, int32_t *perm_slot, int32_t *pos, void *stream);

/*
 * Weight conversion for weight_dtype MOE_DT_F16: count bf16 values at src
 * become IEEE fp16 values at dst, rounded to nearest even: exact for
 * magnitudes in [2^-17, 65504] (a bf16 value has 8 significant bits),
 * smaller ones round to an fp16 subnormal or zero, larger ones overflow to
 * +-inf, NaN stays NaN.  This is the conversion the fp16 GEMMs apply to
 * bf16 weights as they read them.  count is a multiple of 8, both pointers
 * are 16-byte aligned device pointers, dst == src converts in place (other
 * overlaps are rejected).  Returns MOE_ERR_INVALID_ARG on a bad argument.
 */
int moe_convert_bf16_to_f16(const void *src, void *dst, int64_t count, void *stream);

/*
 * Plain device copy dst = src of `bytes` bytes (a multiple of 16; both
 * pointers 16-byte aligned; the ranges must not overlap), with 16-byte
 * loads and stores: the reference kernel for the HBM byte counters
 * (FETCH_SIZE / WRITE_SIZE) and the achievable copy bandwidth that the
 * layer's bandwidth-bound kernels are measured against.
 */
int moe_hbm_copy(void *dst, const void *src, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
