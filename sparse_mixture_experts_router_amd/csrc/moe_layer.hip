// Host side of the C ABI declared in include/moe.h: descriptor validation,
// workspace carving and the launch chain of one layer forward on one stream.
//
// Launch chain (bf16 latent layer), following the layer as described on
// flozi.net "Muse Spark Open: Norm-Preserving Gates Are Not a Norm
// Guarantee", section "Latent experts: normalization happens before the
// weighted sum", and the gate of bobbyburns.tech "816 billion parameters,
// and only 42 billion show up for each token", section "The gate":
//   [input norm] -> router GEMM (fp32 logits) -> top-k + softmax or
//   sigmoid weights -> permutation (counts, scan, stable scatter, tile
//   lists) -> down-projection 8192 -> 4096 [-> latent pre-norm C_pre] ->
//   grouped GEMM1 + SwiGLU -> grouped GEMM2 + per-expert norm partials ->
//   norm + weighted combine -> up-projection 4096 -> 8192 with the linear
//   residual gate out = x + g * y fused into its epilogue, or [output-norm
//   partials ->] output norm + residual gate (linear or alpha/beta).
// The up-projection is linear, so it is applied once to the weighted sum of
// the normalised expert outputs rather than to each of them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "gemm.h"
#include "route.h"

using namespace moe;

namespace {

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Carve {
    size_t total = 0;
    size_t take(size_t bytes) {
        size_t off = total;
        total += align256(bytes);
        return off;
    }
};

struct Layout {
    size_t u, logits, idx, w, counts, offsets, perm_tok, perm_slot, pos, ntiles, tiles_small, tiles_big, tiles_half;
    size_t tiles_tall, perm_scratch, z, act, S, ssq, m, S_out, ssq_out, zq, actq, planes;
    int64_t max_small, max_big, max_half, max_tall;
    size_t total;
};

int64_t small_tile_cap(int64_t TK, int64_t n) { return TK / kSmallBM + n + 1; }
int64_t big_tile_cap(int64_t TK, int64_t n) { return TK / kTileBM + n + 1; }
int64_t half_tile_cap(int64_t n) { return n; }  // at most one per expert
int64_t tall_tile_cap(int64_t n) { return n; }  // at most one per expert

// K slices of the bf16 router GEMM.  It has a single 256-wide column block
// (n <= 256), so a large batch gives only ceil(T / 256) tiles; slicing K
// gives every CU work.  Each slice is a multiple of 512 and adds its
// partial logits into its own fp32 plane; the top-k kernel adds the planes
// in slice order.  Small batches (streaming kernel) are not sliced.
int router_splits(const moe_desc *d) {
    if (d->act_dtype != MOE_DT_BF16 || d->router_dtype != MOE_DT_BF16) return 1;
    // items of the kernel dense_path() picks: 256-row tiles (one column block
    // of 256 experts), or 64-row x 16-expert streaming items; K slices of a
    // multiple of 512 until about one (tiles) or two (streaming) workgroups a CU
    const bool tiled = d->T > 128 && d->n_experts % kTileBN == 0;
    const int64_t items = tiled ? (d->T + kTileBM - 1) / kTileBM : ((d->T + 63) / 64) * (d->n_experts / 16);
    const int64_t target = tiled ? 256 : 512;
    int ks = 1;
    while (items * ks * 2 <= target && d->d_model % (ks * 2 * 512) == 0) ks *= 2;
    return ks;
}

// K slices of the up-projection y = m W_u^T ([T][L] x [d][L]^T) of a few rows
// (32..128) on the bf16 path with bf16 or fp16 weights, the linear residual
// gate or none and no output norm: half-height tiles of 256 columns, K cut in
// two until about one tile per CU (slices a multiple of 512); 1 = the
// streaming kernel instead.  At T = 64 of the 816B-A42B shape this takes the
// up-projection from 37.6 to 27.8 us on one MI355X; the down-projection
// (twice the K, half the columns) measured no faster sliced (28.4 against
// 27.9 us) and stays on the streaming kernel.
int up_splits(const moe_desc *d) {
    if (d->act_dtype != MOE_DT_BF16 || (d->weight_dtype != MOE_DT_BF16 && d->weight_dtype != MOE_DT_F16)) return 1;
    if (d->d_latent == 0 || d->out_norm != MOE_NORM_NONE || d->res_gate == MOE_RES_MUSE) return 1;
    if (d->T < 32 || d->T > 128 || d->d_model % kTileBN) return 1;
    int ks = 1;
    while ((d->d_model / kTileBN) * ks * 2 <= 256 && d->d_latent % (ks * 2 * 512) == 0) ks *= 2;
    return ks;
}

Layout make_layout(const moe_desc *d) {
    Layout L;
    memset(&L, 0, sizeof(L));
    Carve c;
    const int64_t T = d->T, n = d->n_experts, k = d->top_k, TK = T * k;
    const bool bf = d->act_dtype == MOE_DT_BF16;
    const int64_t Dx = d->d_latent ? d->d_latent : d->d_model;  // expert-space width
    const size_t ab = bf ? 2 : 4;                                 // activation bytes
    L.u = (bf && d->in_norm != MOE_NORM_NONE) ? c.take((size_t)T * d->d_model * 2) : 0;
    L.logits = c.take((size_t)router_splits(d) * T * n * 4);
    L.idx = c.take((size_t)TK * 4);
    L.w = c.take((size_t)TK * 4);
    L.counts = c.take((size_t)n * 4);
    L.offsets = c.take((size_t)(n + 1) * 4);
    L.perm_tok = c.take((size_t)TK * 4);
    L.perm_slot = c.take((size_t)TK * 4);
    L.pos = c.take((size_t)TK * 4);
    L.ntiles = c.take(4 * 4);
    L.max_small = small_tile_cap(TK, n);
    L.max_big = big_tile_cap(TK, n);
    L.max_half = half_tile_cap(n);
    L.max_tall = tall_tile_cap(n);
    L.tiles_small = c.take((size_t)L.max_small * sizeof(TileEntry));
    L.tiles_big = c.take((size_t)L.max_big * sizeof(TileEntry));
    L.tiles_half = c.take((size_t)L.max_half * sizeof(TileEntry));
    L.tiles_tall = c.take((size_t)L.max_tall * sizeof(TileEntry));
    L.perm_scratch = c.take((size_t)permute_scratch_ints(T, (int)n) * 4);
    L.z = d->d_latent ? c.take((size_t)T * d->d_latent * 2) : 0;
    L.act = c.take((size_t)TK * d->d_ff * ab);
    L.S = c.take((size_t)TK * Dx * ab);
    L.ssq = (bf && d->expert_norm != MOE_NORM_NONE) ? c.take((size_t)TK * (Dx / 16) * 4) : 0;
    L.m = d->d_latent ? c.take((size_t)T * d->d_latent * 2) : 0;
    const bool onorm = bf && d->out_norm != MOE_NORM_NONE;
    L.S_out = onorm ? c.take((size_t)T * d->d_model * 2) : 0;
    L.ssq_out = onorm ? c.take((size_t)T * (d->d_model / 16) * 4) : 0;
    const bool q8 = bf && d->act_quant == MOE_AQ_MXFP8;
    L.zq = q8 ? c.take((size_t)T * d->d_latent * 33 / 32) : 0;
    L.actq = q8 ? c.take((size_t)TK * d->d_ff * 33 / 32) : 0;
    // fp32 partial sums of the K-sliced up-projection
    const int ku = up_splits(d);
    L.planes = ku > 1 ? c.take((size_t)ku * T * d->d_model * 4) : 0;
    L.total = c.total;
    return L;
}

int check_desc(const moe_desc *d) {
    if (!d) return MOE_ERR_INVALID_ARG;
    if (d->T < 0 || d->d_model <= 0 || d->d_latent < 0 || d->n_experts < 1 || d->top_k < 1 || d->d_ff <= 0)
        return MOE_ERR_INVALID_ARG;
    if (d->n_experts > 256 || d->top_k > d->n_experts || d->top_k > 16) return MOE_ERR_INVALID_ARG;
    if (d->expert_kind != MOE_EXPERT_RELU2 && d->expert_kind != MOE_EXPERT_SWIGLU3) return MOE_ERR_INVALID_ARG;
    if (d->act_dtype != MOE_DT_F32 && d->act_dtype != MOE_DT_BF16) return MOE_ERR_INVALID_ARG;
    if (d->router_dtype != MOE_DT_F32 && d->router_dtype != MOE_DT_BF16) return MOE_ERR_INVALID_ARG;
    if (d->weight_dtype < MOE_DT_F32 || d->weight_dtype > MOE_DT_F16) return MOE_ERR_INVALID_ARG;
    if (d->in_norm < MOE_NORM_NONE || d->in_norm > MOE_NORM_INPUT_SCALED) return MOE_ERR_INVALID_ARG;
    if (d->expert_norm < MOE_NORM_NONE || d->expert_norm > MOE_NORM_INPUT_SCALED) return MOE_ERR_INVALID_ARG;
    if (d->res_gate != MOE_RES_NONE && d->res_gate != MOE_RES_LINEAR && d->res_gate != MOE_RES_MUSE)
        return MOE_ERR_INVALID_ARG;
    if (!(d->eps_in >= 0.f) || !(d->eps_expert >= 0.f)) return MOE_ERR_INVALID_ARG;
    if (d->router_fn != MOE_ROUTER_SOFTMAX && d->router_fn != MOE_ROUTER_SIGMOID) return MOE_ERR_INVALID_ARG;
    if (d->router_fn == MOE_ROUTER_SIGMOID &&
        (d->bias_in_weights || !isfinite(d->router_out_mult) || !isfinite(d->routed_scale)))
        return MOE_ERR_INVALID_ARG;
    if (d->latent_norm < MOE_NORM_NONE || d->latent_norm > MOE_NORM_INPUT_SCALED) return MOE_ERR_INVALID_ARG;
    if (d->out_norm < MOE_NORM_NONE || d->out_norm > MOE_NORM_INPUT_SCALED) return MOE_ERR_INVALID_ARG;
    if (d->latent_norm != MOE_NORM_NONE && (d->d_latent == 0 || !(d->eps_latent >= 0.f))) return MOE_ERR_INVALID_ARG;
    if (d->out_norm != MOE_NORM_NONE && !(d->eps_out >= 0.f)) return MOE_ERR_INVALID_ARG;
    if (d->res_gate == MOE_RES_MUSE && !(d->res_tau > 0.f && isfinite(d->res_tau) && d->res_floor >= 0.f &&
                                         isfinite(d->res_floor)))
        return MOE_ERR_INVALID_ARG;
    if (d->interm_dtype != MOE_DT_F32 && d->interm_dtype != MOE_DT_BF16 && d->interm_dtype != MOE_DT_F16)
        return MOE_ERR_INVALID_ARG;
    if (d->T * d->top_k >= ((int64_t)1 << 31) || d->T >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
    if (d->act_quant != MOE_AQ_NONE && d->act_quant != MOE_AQ_MXFP8) return MOE_ERR_INVALID_ARG;
    if (d->expert_kind == MOE_EXPERT_RELU2 && d->d_latent != 0) return MOE_ERR_INVALID_ARG;
    if (d->act_dtype == MOE_DT_F32) {
        // fp32 path: the small Shazeer layer shape (no latent, no norms).
        if (d->router_dtype != MOE_DT_F32 || d->weight_dtype != MOE_DT_F32) return MOE_ERR_UNSUPPORTED;
        if (d->d_latent != 0 || d->in_norm != MOE_NORM_NONE || d->expert_norm != MOE_NORM_NONE)
            return MOE_ERR_UNSUPPORTED;
        if (d->out_norm != MOE_NORM_NONE || d->res_gate == MOE_RES_MUSE) return MOE_ERR_UNSUPPORTED;
        if (d->act_quant != MOE_AQ_NONE) return MOE_ERR_UNSUPPORTED;
        return MOE_OK;
    }
    // quantized activations: the scaled fp8 x fp4 MFMA path of MXFP4 weights
    if (d->act_quant == MOE_AQ_MXFP8 && d->weight_dtype != MOE_DT_MXFP4) return MOE_ERR_UNSUPPORTED;
    // bf16 path: latent SwiGLU layer on MFMA tiles.
    if (d->router_dtype != MOE_DT_BF16 || d->weight_dtype == MOE_DT_F32) return MOE_ERR_UNSUPPORTED;
    // fp16 weights feed the fp16 GEMMs directly: only with fp16 intermediates
    if (d->weight_dtype == MOE_DT_F16 && d->interm_dtype == MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
    if (d->d_latent == 0 || d->expert_kind != MOE_EXPERT_SWIGLU3) return MOE_ERR_UNSUPPORTED;
    if (d->d_model % 512 || d->d_latent % 512 || d->d_ff % 512 || d->n_experts % 16) return MOE_ERR_UNSUPPORTED;
    // the expert GEMMs address the latent rows they gather with 32-bit offsets
    if (d->T * d->d_latent * 2 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    // the latent pre-norm is the output-scaled form; the output norm and the
    // residual-gate kernel hold a row of at most 8192 values per workgroup
    if (d->latent_norm == MOE_NORM_INPUT_SCALED) return MOE_ERR_UNSUPPORTED;
    if ((d->out_norm != MOE_NORM_NONE || d->res_gate == MOE_RES_MUSE) && d->d_model > 8192) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

inline hipStream_t as_stream(void *s) { return (hipStream_t)s; }

struct Events {
    hipEvent_t *ev;
    hipStream_t s;
    int begin(int stage) { return ev ? (hipEventRecord(ev[2 * stage], s) == hipSuccess ? 0 : MOE_ERR_HIP) : 0; }
    int end(int stage) { return ev ? (hipEventRecord(ev[2 * stage + 1], s) == hipSuccess ? 0 : MOE_ERR_HIP) : 0; }
};

#define MOE_TRY(expr)                                \
    do {                                             \
        if ((expr) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)
#define MOE_TRY_RC(expr)         \
    do {                         \
        int rc_ = (expr);        \
        if (rc_) return rc_;     \
    } while (0)

// Dense C[T][N] = A[T][K] * B[N][K]^T: the streaming kernel for few rows,
// the tiled kernel otherwise.
int dense_path(const GemmArgs &g) { return (g.M <= 128 || g.N % kTileBN != 0) ? PATH_STREAM : PATH_TILE; }

int interm_act(const moe_desc *d) { return d->interm_dtype == MOE_DT_BF16 ? ACT_BF16 : ACT_F16; }

RouterFn router_fn_of(const moe_desc *d) {
    return RouterFn{d->router_fn == MOE_ROUTER_SIGMOID ? kRouterSigmoid : kRouterSoftmax, d->router_out_mult,
                    d->routed_scale};
}

int res_mode_of(const moe_desc *d) {
    return d->res_gate == MOE_RES_MUSE ? kResMuse : d->res_gate == MOE_RES_LINEAR ? kResLinear : kResNone;
}

int forward_bf16(const moe_desc *d, const void *x, const void *router_w, const void *down_w, const void *w1,
                 const void *w2, const void *up_w, const moe_gains *gains, void *out, uint8_t *ws, const Layout &L,
                 moe_debug *dbg, hipStream_t s) {
    const int64_t T = d->T, D = d->d_model, Lw = d->d_latent, n = d->n_experts, k = d->top_k, F = d->d_ff;
    const int64_t TK = T * k;
    const bool mx = d->weight_dtype == MOE_DT_MXFP4;
    const int at = interm_act(d);
    // operand types of the GEMMs on the fp16 intermediates (expert GEMMs and
    // the up-projection): fp16 weights need no conversion; down_w is bf16
    // in every format but MXFP4
    const int wat = d->weight_dtype == MOE_DT_F16 ? ACT_F16_W16 : at;
    Events ev{dbg ? (hipEvent_t *)dbg->stage_events : nullptr, s};

    const uint16_t *xb = (const uint16_t *)x;
    const uint16_t *u = xb;
    if (d->in_norm != MOE_NORM_NONE) {
        MOE_TRY_RC(ev.begin(MOE_STAGE_IN_NORM));
        uint16_t *ub = (uint16_t *)(ws + L.u);
        MOE_TRY(launch_rmsnorm(xb, gains->gamma_in, ub, T, D, d->eps_in,
                               d->in_norm == MOE_NORM_CENTERED ? 1 : 2, ACT_BF16, s));
        MOE_TRY_RC(ev.end(MOE_STAGE_IN_NORM));
        u = ub;
    }
    float *logits = (float *)(ws + L.logits);
    int32_t *idx = (int32_t *)(ws + L.idx);
    float *wts = (float *)(ws + L.w);
    int32_t *counts = (int32_t *)(ws + L.counts), *offsets = (int32_t *)(ws + L.offsets);
    int32_t *perm_tok = (int32_t *)(ws + L.perm_tok), *perm_slot = (int32_t *)(ws + L.perm_slot);
    int32_t *pos = (int32_t *)(ws + L.pos), *ntiles = (int32_t *)(ws + L.ntiles);
    TileEntry *tiles_small = (TileEntry *)(ws + L.tiles_small), *tiles_big = (TileEntry *)(ws + L.tiles_big);
    TileEntry *tiles_half = (TileEntry *)(ws + L.tiles_half), *tiles_tall = (TileEntry *)(ws + L.tiles_tall);
    int32_t *perm_scratch = (int32_t *)(ws + L.perm_scratch);
    uint16_t *z = (uint16_t *)(ws + L.z), *act = (uint16_t *)(ws + L.act), *S = (uint16_t *)(ws + L.S);
    uint16_t *m = (uint16_t *)(ws + L.m);
    float *ssq = L.ssq ? (float *)(ws + L.ssq) : nullptr;

    // Router logits (fp32) = u W_r^T.
    MOE_TRY_RC(ev.begin(MOE_STAGE_ROUTER));
    {
        GemmArgs g{};
        g.A = u;
        g.lda = D;
        g.B = router_w;
        g.b_rows_total = n;
        g.N = n;
        g.K = D;
        g.M = T;
        g.C = logits;
        g.ldc = n;
        g.ksplit = router_splits(d);
        MOE_TRY(launch_router_gemm(g, dense_path(g), s));
    }
    MOE_TRY_RC(ev.end(MOE_STAGE_ROUTER));

    MOE_TRY_RC(ev.begin(MOE_STAGE_TOPK));
    MOE_TRY(launch_topk(logits, router_splits(d), gains ? gains->router_bias : nullptr, T, (int)n, (int)k,
                        d->bias_in_weights, router_fn_of(d), idx, wts, dbg ? dbg->logits : nullptr, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_TOPK));

    // Experts with up to small_max tokens are streamed (weight-bandwidth
    // bound); heavier experts use the tiled kernel.
    const int64_t avg = (TK + n - 1) / n;
    const int small_max = (avg <= 32) ? (int)(T < 0x7fffffff ? T : 0x7fffffff) : 32;
    const bool any_big = T > small_max;
    MOE_TRY_RC(ev.begin(MOE_STAGE_PERMUTE));
    MOE_TRY(launch_permute(idx, T, (int)k, (int)n, counts, offsets, perm_tok, perm_slot, pos, tiles_small, tiles_big,
                           tiles_half, tiles_tall, ntiles, small_max, perm_scratch, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_PERMUTE));

    // z = u W_d^T (bf16).
    MOE_TRY_RC(ev.begin(MOE_STAGE_DOWN));
    {
        GemmArgs g{};
        g.A = u;
        g.lda = D;
        g.B = down_w;
        g.b_rows_total = Lw;
        g.N = Lw;
        g.K = D;
        g.M = T;
        g.C = z;
        g.ldc = Lw;
        MOE_TRY(launch_down_gemm(g, dense_path(g), mx, at, s));
    }
    if (d->latent_norm != MOE_NORM_NONE)  // z = C_pre(z), in place, in the intermediate type
        MOE_TRY(launch_rmsnorm(z, gains ? gains->gamma_latent : nullptr, z, T, Lw, d->eps_latent, 1, at, s));
    // MXFP8 activations: the expert GEMMs read the quantized z
    const bool q8 = d->act_quant == MOE_AQ_MXFP8;
    uint8_t *zq = q8 ? ws + L.zq : nullptr, *actq = q8 ? ws + L.actq : nullptr;
    if (q8) MOE_TRY(launch_mxfp8_rows(z, T, Lw, at, zq, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_DOWN));
    auto gemm1 = [&](const GemmArgs &g, int path) {
        return q8 ? launch_gemm1_q8(g, path, at, s) : launch_gemm1(g, path, mx, wat, s);
    };
    auto gemm2 = [&](const GemmArgs &g, int path, bool norm) {
        return q8 ? launch_gemm2_q8(g, path, norm, s) : launch_gemm2(g, path, mx, wat, norm, s);
    };

    auto grouped = [&](GemmArgs &g) {
        g.counts = counts;
        g.offsets = offsets;
    };
    // GEMM1: act[p] = silu(z[tok(p)] Wg_e^T) * (z[tok(p)] Wu_e^T).
    MOE_TRY_RC(ev.begin(MOE_STAGE_GEMM1));
    {
        GemmArgs g{};
        g.A = z;
        g.a_gather = perm_tok;
        g.lda = Lw;
        g.B = w1;
        g.b_rows_total = n * 2 * F;
        g.b_group_rows = 2 * F;
        g.N = F;
        g.K = Lw;
        g.C = act;
        g.ldc = F;
        g.A8 = zq;
        g.A8s = q8 ? zq + (size_t)T * Lw : nullptr;
        grouped(g);
        g.tiles = tiles_small;
        g.ntiles = ntiles;
        g.max_tiles = (int32_t)L.max_small;
        MOE_TRY(gemm1(g, PATH_STREAM));
        if (any_big) {
            g.tiles = tiles_big;
            g.ntiles = ntiles + 1;
            g.max_tiles = (int32_t)L.max_big;
            MOE_TRY(gemm1(g, PATH_TILE));
            g.tiles = tiles_half;
            g.ntiles = ntiles + 2;
            g.max_tiles = (int32_t)L.max_half;
            MOE_TRY(gemm1(g, PATH_HALF));
            g.tiles = tiles_tall;
            g.ntiles = ntiles + 3;
            g.max_tiles = (int32_t)L.max_tall;
            MOE_TRY(gemm1(g, PATH_TALL));
        }
        // MXFP8 activations: GEMM2 reads the quantized SwiGLU output
        if (q8) MOE_TRY(launch_mxfp8_rows(act, TK, F, at, actq, s));
    }
    MOE_TRY_RC(ev.end(MOE_STAGE_GEMM1));

    // GEMM2: S[p] = bf16((1+gamma) * act[p] W2_e^T) and per-16-column sums of squares.
    const bool norm2 = d->expert_norm != MOE_NORM_NONE;
    MOE_TRY_RC(ev.begin(MOE_STAGE_GEMM2));
    {
        GemmArgs g{};
        g.A = act;
        g.lda = F;
        g.B = w2;
        g.b_rows_total = n * Lw;
        g.b_group_rows = Lw;
        g.N = Lw;
        g.K = F;
        g.C = S;
        g.ldc = Lw;
        g.gamma = gains ? gains->gamma_expert : nullptr;
        g.ssq = ssq;
        g.nparts = (int32_t)(Lw / 16);
        g.norm_round = d->expert_norm == MOE_NORM_INPUT_SCALED ? 1 : 0;
        g.A8 = actq;
        g.A8s = q8 ? actq + (size_t)TK * F : nullptr;
        grouped(g);
        g.tiles = tiles_small;
        g.ntiles = ntiles;
        g.max_tiles = (int32_t)L.max_small;
        MOE_TRY(gemm2(g, PATH_STREAM, norm2));
        if (any_big) {
            g.tiles = tiles_big;
            g.ntiles = ntiles + 1;
            g.max_tiles = (int32_t)L.max_big;
            MOE_TRY(gemm2(g, PATH_TILE, norm2));
            g.tiles = tiles_half;
            g.ntiles = ntiles + 2;
            g.max_tiles = (int32_t)L.max_half;
            MOE_TRY(gemm2(g, PATH_HALF, norm2));
            g.tiles = tiles_tall;
            g.ntiles = ntiles + 3;
            g.max_tiles = (int32_t)L.max_tall;
            MOE_TRY(gemm2(g, PATH_TALL, norm2));
        }
    }
    MOE_TRY_RC(ev.end(MOE_STAGE_GEMM2));

    MOE_TRY_RC(ev.begin(MOE_STAGE_COMBINE));
    MOE_TRY(launch_combine(S, ssq, pos, wts, T, Lw, (int)(Lw / 16), d->eps_expert, (int)k, at, m, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_COMBINE));

    // y = m W_u^T.  The linear gate without an output norm is fused into the
    // epilogue (out = x + g * y); otherwise the epilogue stores y (fp32, in
    // out) or the output norm's bf16 (1 + gamma) y and partial sums, and the
    // residual-gate kernel finishes the row.
    const bool fused = d->out_norm == MOE_NORM_NONE && d->res_gate != MOE_RES_MUSE;
    MOE_TRY_RC(ev.begin(MOE_STAGE_UP));
    {
        GemmArgs g{};
        g.A = m;
        g.lda = Lw;
        g.B = up_w;
        g.b_rows_total = D;
        g.N = D;
        g.K = Lw;
        g.M = T;
        g.C = out;
        g.ldc = D;
        const int ks = up_splits(d);
        if (ks > 1) {
            const bool lin = d->res_gate == MOE_RES_LINEAR;
            g.C = ws + L.planes;
            g.ksplit = ks;
            MOE_TRY(launch_dense_split(g, wat, s));
            MOE_TRY(launch_split_reduce((const float *)(ws + L.planes), ks, T, D, lin ? EPI_RESID : EPI_F32, out,
                                        lin ? xb : nullptr, lin ? gains->res_gate : nullptr,
                                        lin && dbg ? dbg->y : nullptr, s));
            if (!lin && dbg && dbg->y)
                MOE_TRY(hipMemcpyAsync(dbg->y, out, (size_t)T * D * 4, hipMemcpyDeviceToDevice, s));
        } else if (fused && d->res_gate == MOE_RES_LINEAR) {
            g.resid = xb;
            g.gate = gains->res_gate;
            g.y = dbg ? dbg->y : nullptr;
            MOE_TRY(launch_up_gemm(g, dense_path(g), mx, wat, EPI_RESID, s));
        } else if (d->out_norm != MOE_NORM_NONE) {
            g.C = ws + L.S_out;
            g.gamma = gains ? gains->gamma_out : nullptr;
            g.ssq = (float *)(ws + L.ssq_out);
            g.nparts = (int32_t)(D / 16);
            g.norm_round = d->out_norm == MOE_NORM_INPUT_SCALED ? 1 : 0;
            MOE_TRY(launch_up_gemm(g, dense_path(g), mx, wat, EPI_NORM, s));
        } else {
            MOE_TRY(launch_up_gemm(g, dense_path(g), mx, wat, EPI_F32, s));
            if (fused && dbg && dbg->y)
                MOE_TRY(hipMemcpyAsync(dbg->y, out, (size_t)T * D * 4, hipMemcpyDeviceToDevice, s));
        }
    }
    MOE_TRY_RC(ev.end(MOE_STAGE_UP));
    if (!fused) {
        MOE_TRY_RC(ev.begin(MOE_STAGE_RESGATE));
        const bool onorm = d->out_norm != MOE_NORM_NONE;
        MOE_TRY(launch_resgate(onorm ? (const uint16_t *)(ws + L.S_out) : nullptr,
                               onorm ? (const float *)(ws + L.ssq_out) : nullptr, (int)(D / 16), d->eps_out, xb,
                               gains ? gains->res_gate : nullptr, res_mode_of(d), d->res_tau, d->res_floor, T, D,
                               (float *)out, dbg ? dbg->y : nullptr, s));
        MOE_TRY_RC(ev.end(MOE_STAGE_RESGATE));
    }

    if (dbg) {
        if (dbg->topk_idx) MOE_TRY(hipMemcpyAsync(dbg->topk_idx, idx, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->topk_w) MOE_TRY(hipMemcpyAsync(dbg->topk_w, wts, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->expert_counts) MOE_TRY(hipMemcpyAsync(dbg->expert_counts, counts, n * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->expert_offsets)
            MOE_TRY(hipMemcpyAsync(dbg->expert_offsets, offsets, (n + 1) * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->perm_tok) MOE_TRY(hipMemcpyAsync(dbg->perm_tok, perm_tok, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->perm_slot) MOE_TRY(hipMemcpyAsync(dbg->perm_slot, perm_slot, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->pos) MOE_TRY(hipMemcpyAsync(dbg->pos, pos, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->z) MOE_TRY(hipMemcpyAsync(dbg->z, z, (size_t)T * Lw * 2, hipMemcpyDeviceToDevice, s));
        if (dbg->act) MOE_TRY(hipMemcpyAsync(dbg->act, act, (size_t)TK * F * 2, hipMemcpyDeviceToDevice, s));
        if (dbg->S) MOE_TRY(hipMemcpyAsync(dbg->S, S, (size_t)TK * Lw * 2, hipMemcpyDeviceToDevice, s));
        if (dbg->ssq && ssq)
            MOE_TRY(hipMemcpyAsync(dbg->ssq, ssq, (size_t)TK * (Lw / 16) * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->m) MOE_TRY(hipMemcpyAsync(dbg->m, m, (size_t)T * Lw * 2, hipMemcpyDeviceToDevice, s));
        if (dbg->u) MOE_TRY(hipMemcpyAsync(dbg->u, u, (size_t)T * D * 2, hipMemcpyDeviceToDevice, s));
        if (dbg->zq && q8)
            MOE_TRY(hipMemcpyAsync(dbg->zq, zq, (size_t)T * Lw * 33 / 32, hipMemcpyDeviceToDevice, s));
        if (dbg->actq && q8)
            MOE_TRY(hipMemcpyAsync(dbg->actq, actq, (size_t)TK * F * 33 / 32, hipMemcpyDeviceToDevice, s));
    }
    return MOE_OK;
}

int forward_f32(const moe_desc *d, const void *x, const void *router_w, const void *w1, const void *w2,
                const moe_gains *gains, void *out, uint8_t *ws, const Layout &L, moe_debug *dbg, hipStream_t s) {
    const int64_t T = d->T, D = d->d_model, n = d->n_experts, k = d->top_k, F = d->d_ff, TK = T * k;
    Events ev{dbg ? (hipEvent_t *)dbg->stage_events : nullptr, s};
    float *logits = (float *)(ws + L.logits);
    int32_t *idx = (int32_t *)(ws + L.idx);
    float *wts = (float *)(ws + L.w);
    int32_t *counts = (int32_t *)(ws + L.counts), *offsets = (int32_t *)(ws + L.offsets);
    int32_t *perm_tok = (int32_t *)(ws + L.perm_tok), *perm_slot = (int32_t *)(ws + L.perm_slot);
    int32_t *pos = (int32_t *)(ws + L.pos);
    float *act = (float *)(ws + L.act), *S = (float *)(ws + L.S);

    MOE_TRY_RC(ev.begin(MOE_STAGE_ROUTER));
    MOE_TRY(launch_router_f32((const float *)x, (const float *)router_w, T, (int)n, D, logits, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_ROUTER));
    MOE_TRY_RC(ev.begin(MOE_STAGE_TOPK));
    MOE_TRY(launch_topk(logits, 1, gains ? gains->router_bias : nullptr, T, (int)n, (int)k, d->bias_in_weights,
                        router_fn_of(d), idx, wts, dbg ? dbg->logits : nullptr, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_TOPK));
    MOE_TRY_RC(ev.begin(MOE_STAGE_PERMUTE));
    MOE_TRY(launch_permute(idx, T, (int)k, (int)n, counts, offsets, perm_tok, perm_slot, pos, nullptr, nullptr,
                           nullptr, nullptr, nullptr, 0, (int32_t *)(ws + L.perm_scratch), s));
    MOE_TRY_RC(ev.end(MOE_STAGE_PERMUTE));
    MOE_TRY_RC(ev.begin(MOE_STAGE_GEMM1));
    MOE_TRY(launch_expert1_f32((const float *)x, (const float *)w1, perm_tok, offsets, (int)n, TK, F, D,
                               d->expert_kind == MOE_EXPERT_SWIGLU3, act, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_GEMM1));
    MOE_TRY_RC(ev.begin(MOE_STAGE_GEMM2));
    MOE_TRY(launch_expert2_f32(act, (const float *)w2, offsets, (int)n, TK, F, D, S, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_GEMM2));
    MOE_TRY_RC(ev.begin(MOE_STAGE_COMBINE));
    MOE_TRY(launch_combine_f32(S, pos, wts, (const float *)x,
                               d->res_gate == MOE_RES_LINEAR ? gains->res_gate : nullptr, T, (int)k, D, (float *)out,
                               dbg ? dbg->y : nullptr, s));
    MOE_TRY_RC(ev.end(MOE_STAGE_COMBINE));
    if (dbg) {
        if (dbg->topk_idx) MOE_TRY(hipMemcpyAsync(dbg->topk_idx, idx, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->topk_w) MOE_TRY(hipMemcpyAsync(dbg->topk_w, wts, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->expert_counts) MOE_TRY(hipMemcpyAsync(dbg->expert_counts, counts, n * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->expert_offsets)
            MOE_TRY(hipMemcpyAsync(dbg->expert_offsets, offsets, (n + 1) * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->perm_tok) MOE_TRY(hipMemcpyAsync(dbg->perm_tok, perm_tok, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->perm_slot) MOE_TRY(hipMemcpyAsync(dbg->perm_slot, perm_slot, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->pos) MOE_TRY(hipMemcpyAsync(dbg->pos, pos, TK * 4, hipMemcpyDeviceToDevice, s));
        if (dbg->u) MOE_TRY(hipMemcpyAsync(dbg->u, x, (size_t)T * D * 4, hipMemcpyDeviceToDevice, s));
    }
    return MOE_OK;
}

// Clears an error left pending by an earlier HIP call of the calling thread,
// so the launchers' hipGetLastError reports their own launches only.
inline void clear_stale_error() { (void)hipGetLastError(); }

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of moe_layer_forward_static: the workspace of callers that
// cannot allocate.  Every device the library runs on holds its own copy
// until the process ends.  Host code never uses the name `scratch` as an
// address (on the host it names a stand-in, not device memory): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept in static_scratch_ptr.
// ---------------------------------------------------------------------------
static_assert(MOE_STATIC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");
__device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int static_scratch_ptr(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_error_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOE_ERR_HIP: return "HIP error";
        case MOE_ERR_STATIC_SCRATCH_TOO_SMALL: return "batch needs more than the static scratch";
    }
    return "unknown status";
}

int moe_validate(const moe_desc *desc) { return check_desc(desc); }

size_t moe_workspace_bytes(const moe_desc *desc) {
    if (check_desc(desc) != MOE_OK) return 0;
    return make_layout(desc).total;
}

int moe_layer_forward(const moe_desc *d, const void *x, const void *router_w, const void *down_w,
                      const void *expert_w1, const void *expert_w2, const void *up_w, const moe_gains *gains,
                      void *out, void *workspace, size_t workspace_bytes, moe_debug *dbg, void *stream) {
    int rc = check_desc(d);
    if (rc != MOE_OK) return rc;
    if (d->T == 0) return MOE_OK;  // nothing to read or write: pointers may be NULL
    if (!x || !router_w || !expert_w1 || !expert_w2 || !out) return MOE_ERR_INVALID_ARG;
    if (d->d_latent && (!down_w || !up_w)) return MOE_ERR_INVALID_ARG;
    if (d->res_gate != MOE_RES_NONE && (!gains || !gains->res_gate)) return MOE_ERR_INVALID_ARG;
    if (d->in_norm != MOE_NORM_NONE && !gains) return MOE_ERR_INVALID_ARG;
    Layout L = make_layout(d);
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || ((uintptr_t)workspace & 255)) return MOE_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    clear_stale_error();
    if (d->act_dtype == MOE_DT_BF16)
        return forward_bf16(d, x, router_w, down_w, expert_w1, expert_w2, up_w, gains, out, (uint8_t *)workspace, L,
                            dbg, s);
    return forward_f32(d, x, router_w, expert_w1, expert_w2, gains, out, (uint8_t *)workspace, L, dbg, s);
}

int moe_layer_forward_static(const moe_desc *d, const void *x, const void *router_w, const void *down_w,
                             const void *expert_w1, const void *expert_w2, const void *up_w,
                             const moe_gains *gains, void *out, moe_debug *dbg, void *stream) {
    int rc = check_desc(d);
    if (rc != MOE_OK) return rc;
    if (d->T == 0) return MOE_OK;
    const size_t need = make_layout(d).total;
    if (need > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_STATIC_SCRATCH_TOO_SMALL;
    void *ws = nullptr;
    clear_stale_error();
    rc = static_scratch_ptr(&ws);
    if (rc != MOE_OK) return rc;
    return moe_layer_forward(d, x, router_w, down_w, expert_w1, expert_w2, up_w, gains, out, ws,
                             MOE_STATIC_SCRATCH_BYTES, dbg, stream);
}

size_t moe_router_workspace_bytes(const moe_desc *d) {
    if (check_desc(d) != MOE_OK) return 0;
    return align256((size_t)router_splits(d) * d->T * d->n_experts * 4);
}

int moe_router_topk(const moe_desc *d, const void *u, const void *router_w, const float *router_bias,
                    int32_t *topk_idx, float *topk_w, float *logits, void *workspace, size_t workspace_bytes,
                    void *stream) {
    int rc = check_desc(d);
    if (rc != MOE_OK) return rc;
    if (!u || !router_w || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    // the K-sliced router needs the workspace for its partial planes; with
    // logits given and no workspace it runs unsliced straight into them
    float *lg = logits;
    int ks = 1;
    if (workspace && workspace_bytes >= moe_router_workspace_bytes(d)) {
        lg = (float *)workspace;
        ks = router_splits(d);
    } else if (!lg) {
        if (workspace_bytes < moe_router_workspace_bytes(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
        return MOE_ERR_INVALID_ARG;
    }
    if (d->T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    clear_stale_error();
    if (d->router_dtype == MOE_DT_F32) {
        MOE_TRY(launch_router_f32((const float *)u, (const float *)router_w, d->T, (int)d->n_experts, d->d_model, lg,
                                  s));
    } else {
        GemmArgs g{};
        g.A = (const uint16_t *)u;
        g.lda = d->d_model;
        g.B = router_w;
        g.b_rows_total = d->n_experts;
        g.N = d->n_experts;
        g.K = d->d_model;
        g.M = d->T;
        g.C = lg;
        g.ldc = d->n_experts;
        g.ksplit = ks;
        MOE_TRY(launch_router_gemm(g, dense_path(g), s));
    }
    MOE_TRY(launch_topk(lg, ks, router_bias, d->T, (int)d->n_experts, (int)d->top_k, d->bias_in_weights,
                        router_fn_of(d), topk_idx, topk_w, lg == logits ? nullptr : logits, s));
    return MOE_OK;
}

int moe_permute(int64_t T, int64_t k, int64_t n, const int32_t *topk_idx, int32_t *counts, int32_t *offsets,
                int32_t *perm_tok, int32_t *perm_slot, int32_t *pos, void *stream) {
    if (T < 0 || k < 1 || n < 1 || n > 256 || k > n || T * k >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
    if (!topk_idx || !counts || !offsets || !perm_tok || !perm_slot || !pos) return MOE_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    clear_stale_error();
    MOE_TRY(launch_permute(topk_idx, T, (int)k, (int)n, counts, offsets, perm_tok, perm_slot, pos, nullptr, nullptr,
                           nullptr, nullptr, nullptr, 0, nullptr, s));
    return MOE_OK;
}

int moe_convert_bf16_to_f16(const void *src, void *dst, int64_t count, void *stream) {
    if (count < 0 || (count & 7) || (count && (!dst || !src)) || (((uintptr_t)dst | (uintptr_t)src) & 15))
        return MOE_ERR_INVALID_ARG;
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst, bytes = (uintptr_t)count * 2;
    if (a != b && a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // partial overlap
    clear_stale_error();
    MOE_TRY(launch_bf16_to_f16(src, dst, count, as_stream(stream)));
    return MOE_OK;
}

int moe_hbm_copy(void *dst, const void *src, size_t bytes, void *stream) {
    if ((bytes & 15) || (bytes && (!dst || !src)) || (((uintptr_t)dst | (uintptr_t)src) & 15)) return MOE_ERR_INVALID_ARG;
    clear_stale_error();
    MOE_TRY(launch_copy16(src, dst, (int64_t)bytes, as_stream(stream)));
    return MOE_OK;
}

}  // extern "C"
