// Launchers of the non-GEMM kernels of the MoE layer (see route.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace moe {

// Rows of stored type `it` (ACT_BF16 / ACT_F16), same type out; u may equal x.
// mode 1: C_gamma (u = (1+g) x / rms(x)); mode 2: I_gamma (s = rnd((1+g) x), u = s / rms(s)).
hipError_t launch_rmsnorm(const uint16_t *x, const float *gamma, uint16_t *u, int64_t T, int64_t d, float eps,
                          int mode, int it, hipStream_t s);

// Router function of the top-k stage.
constexpr int kRouterSoftmax = 0, kRouterSigmoid = 1;
struct RouterFn {
    int fn;          // kRouterSoftmax or kRouterSigmoid
    float out_mult;  // sigmoid: logit multiplier
    float rsf;       // sigmoid: routed scaling factor
};
// logits: ks planes of [T][n] fp32 partial sums (over disjoint K slices),
// added in plane order; lout (may be NULL) receives the summed logits.
hipError_t launch_topk(const float *logits, int ks, const float *bias, int64_t T, int n, int k, int bias_in_weights,
                       const RouterFn &rf, int32_t *idx, float *w, float *lout, hipStream_t s);
// Experts with 1..small_max tokens go to the small-tile list (kSmallBM rows
// per tile).  Heavier ones get one tile when it holds them (half-height list
// up to kHalfBM rows, full list up to kTileBM, tall list up to kTallBM), else
// full tiles of kTileBM rows plus, for a remainder of at most kHalfBM rows,
// a half-height tile.  ntiles[0..3] receive the four list lengths.  With scratch (permute_scratch_ints(T, n)
// ints) and T >= kPermMultiMinT the work spreads over chunks of tokens;
// otherwise one workgroup does it.
constexpr int64_t kPermMultiMinT = 1024;
int64_t permute_scratch_ints(int64_t T, int n);
hipError_t launch_permute(const int32_t *idx, int64_t T, int k, int n, int32_t *counts, int32_t *offsets,
                          int32_t *perm_tok, int32_t *perm_slot, int32_t *pos, TileEntry *tiles_small,
                          TileEntry *tiles_big, TileEntry *tiles_half, TileEntry *tiles_tall, int32_t *ntiles,
                          int small_max, int32_t *scratch, hipStream_t s);
// m in activation type `ot` (ACT_BF16 / ACT_F16).
hipError_t launch_combine(const uint16_t *S, const float *ssq, const int32_t *pos, const float *w, int64_t T,
                          int64_t L, int nparts, float eps, int k, int ot, uint16_t *m, hipStream_t s);

// Branch output norm + residual gate.  S != NULL: b = S * rsqrt(sum of the
// row's nparts partial sums / d + eps) (S bf16 [T][d], ssq [T][nparts]);
// S == NULL: b = out (fp32 y, overwritten).  out = b, x + g b (kResLinear)
// or alpha x + beta b (kResMuse, temperature tau, floor floor_); ydbg (may
// be NULL) receives b.  d % 8 == 0 and d <= 8192.
constexpr int kResNone = 0, kResLinear = 1, kResMuse = 2;
hipError_t launch_resgate(const uint16_t *S, const float *ssq, int nparts, float eps, const uint16_t *x,
                          const float *g, int res, float tau, float floor_, int64_t T, int64_t d, float *out,
                          float *ydbg, hipStream_t s);

// dst = src, 16 bytes per lane per access (bytes: multiple of 16).
hipError_t launch_copy16(const void *src, void *dst, int64_t bytes, hipStream_t s);
// count bf16 values (a multiple of 8, 16-byte aligned) -> fp16; dst may equal src.
hipError_t launch_bf16_to_f16(const void *src, void *dst, int64_t count, hipStream_t s);

hipError_t launch_router_f32(const float *x, const float *W, int64_t T, int n, int64_t d, float *logits,
                             hipStream_t s);
hipError_t launch_expert1_f32(const float *x, const float *W1, const int32_t *perm_tok, const int32_t *offsets, int n,
                              int64_t TK, int64_t F, int64_t din, int swiglu, float *act, hipStream_t s);
hipError_t launch_expert2_f32(const float *act, const float *W2, const int32_t *offsets, int n, int64_t TK, int64_t F,
                              int64_t dout, float *S, hipStream_t s);
hipError_t launch_combine_f32(const float *S, const int32_t *pos, const float *w, const float *x, const float *gate,
                              int64_t T, int k, int64_t d, float *out, float *y, hipStream_t s);

}  // namespace moe
