// Arguments and launchers of the layer's MFMA GEMMs: C = A * B^T with A rows
// of activations (bf16 or fp16) and B rows of bf16 or MXFP4 weights (both
// with the reduction dimension K contiguous), fp32 accumulation, fused
// epilogues.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Activation (MFMA input) types of the layer's GEMMs.
// Operand types of an MFMA GEMM (template parameter AT) and storage types of
// activations (OT): bf16 activations with bf16 weights; fp16 activations
// with bf16 or MXFP4 weights converted to fp16 as they are read; fp16
// activations with weights already stored as fp16 (AT only); MXFP8
// activations (E4M3 codes with one E8M0 scale per 32 along K) with MXFP4
// weights (AT only): the scaled fp8 x fp4 MFMA on large tiles, both operands
// decoded to bf16 (exactly) on the streaming kernel.
enum ActType : int { ACT_BF16 = 0, ACT_F16 = 1, ACT_F16_W16 = 2, ACT_Q8 = 3 };

enum Epi : int {
    EPI_F32 = 0,     // C[p][n] = acc (fp32)
    EPI_ACT = 1,     // C[p][n] = act(acc), in the output activation type
    EPI_SWIGLU = 2,  // C[p][j] = act(silu(acc[j]) * acc[F + j]); B holds gate rows then up rows
    EPI_NORM = 3,    // C[p][n] = s = bf16((1 + gamma[n]) * acc); ssq[p][n/16] = sums of squares per 16 columns
    EPI_RESID = 4    // out[p][n] = x[p][n] + gate[n] * acc (fp32); y[p][n] = acc when y != NULL
};

struct TileEntry {  // one M-tile of a grouped GEMM: expert e, rows m0 .. of its segment
    int32_t e;
    int32_t m0;
    int32_t p0;      // its first permuted row: the expert's offset + m0
    int32_t mcount;  // its valid rows (1 .. the list's tile height)
};

struct GemmArgs {
    // A: activation rows with leading dimension lda.  Grouped GEMMs index rows
    // by permuted position p; a_gather (may be NULL) maps p to the A row.
    const uint16_t *A;
    const int32_t *a_gather;
    int64_t lda;
    // B: [b_rows_total][K] bf16, or one MXFP4 buffer of b_rows_total rows.
    const void *B;
    int64_t b_rows_total;
    int64_t b_group_rows;  // rows of B per expert (grouped), 0 when dense
    int64_t N;             // output columns (EPI_SWIGLU: F, and B has 2F rows per expert)
    int64_t K;
    // rows
    int64_t M;             // dense: number of rows (tiles = ceil(M / BM))
    const TileEntry *tiles; // grouped: tile list and its device-side length
    const int32_t *ntiles;
    const int32_t *counts;  // grouped: tokens per expert
    const int32_t *offsets; // grouped: first permuted row of each expert
    int32_t max_tiles;      // grouped: capacity of the tile list
    // epilogue
    void *C;
    int64_t ldc;
    const float *gamma;    // EPI_NORM gain (NULL = 1)
    float *ssq;            // EPI_NORM partial sums of squares [rows][nparts]
    int32_t nparts;
    int32_t norm_round;    // EPI_NORM: 1 squares the bf16-rounded scaled value (input-scaled norm)
    const uint16_t *resid; // EPI_RESID: x rows (bf16), leading dimension N
    const float *gate;     // EPI_RESID: g [N]
    float *y;              // EPI_RESID: optional y [rows][N]
    // dense EPI_F32 tiles on bf16 weights: ksplit > 1 splits K into that many
    // equal slices (each a multiple of 512), slice s adding its partial sums
    // into plane s of C ([ksplit][M][ldc]); 0 or 1 = no split
    int32_t ksplit;
    // ACT_Q8: the A rows as E4M3 codes [rows][K] (row stride K bytes) and their
    // E8M0 scales [rows][K/32], row-indexed like A (gathered through a_gather
    // or contiguous); A itself is not read
    const uint8_t *A8;
    const uint8_t *A8s;
};

constexpr int kTileBM = 256;      // rows per tile of the large-tile kernel (and of its grouped lists)
constexpr int kHalfBM = 128;      // rows per tile of its half-height variant (expert remainders)
constexpr int kTallBM = 320;      // rows of its tall variant (one tile for an expert with 257..320 rows)
constexpr int kTileBN = 256;      // B rows per tile (SWIGLU: 128 gate + 128 up -> 128 outputs)
constexpr int kSmallBM = 16;      // rows per tile of the streaming kernel's grouped lists

// Kernel choice for a launch.
enum GemmPath : int { PATH_STREAM = 0, PATH_TILE = 1, PATH_HALF = 2, PATH_TALL = 3 };

// Router logits: dense, A = u (bf16), B = router weight (bf16), fp32 out.
hipError_t launch_router_gemm(const GemmArgs &a, int path, hipStream_t s);
// Down-projection: dense, A = u (bf16), output z in activation type `ot`.
hipError_t launch_down_gemm(const GemmArgs &a, int path, bool mx, int ot, hipStream_t s);
// Expert GEMM1 + SwiGLU: grouped, A = z in activation type `at`, output in `at`.
hipError_t launch_gemm1(const GemmArgs &a, int path, bool mx, int at, hipStream_t s);
// Expert GEMM2: grouped, A = act in `at`; EPI_NORM (bf16 S + partial sums) or EPI_ACT with bf16 S.
hipError_t launch_gemm2(const GemmArgs &a, int path, bool mx, int at, bool norm, hipStream_t s);
// Expert GEMM1 + SwiGLU and GEMM2 on MXFP8 activations (A8, A8s) and MXFP4
// weights; GEMM1's output in `ot` (ACT_F16 / ACT_BF16), GEMM2's as launch_gemm2.
hipError_t launch_gemm1_q8(const GemmArgs &a, int path, int ot, hipStream_t s);
hipError_t launch_gemm2_q8(const GemmArgs &a, int path, bool norm, hipStream_t s);
// MXFP8 quantization of 16-bit activation rows (ACT_BF16 or ACT_F16 storage
// `it`): x [rows][K] (K % 32 == 0) -> E4M3 codes q [rows][K], then E8M0 scales
// [rows][K/32] at q + rows * K (one buffer, the layout of an MXFP4 matrix).
hipError_t launch_mxfp8_rows(const uint16_t *x, int64_t rows, int64_t K, int it, uint8_t *q, hipStream_t s);
// Up-projection: dense, A = m in `at`; epi = EPI_RESID, EPI_F32, or EPI_NORM
// (bf16 (1 + gamma) y and per-16-column sums of squares for the output norm).
hipError_t launch_up_gemm(const GemmArgs &a, int path, bool mx, int at, int epi, hipStream_t s);

// Dense projection of a few rows (at most 128) on half-height tiles (128 x
// 256) with K cut into a.ksplit >= 2 slices of a multiple of 512: slice s
// stores its partial sums into fp32 plane s of C ([ksplit][M][ldc], ldc = N).
// A in `at`, bf16 or fp16 weights.  launch_split_reduce finishes the sums.
hipError_t launch_dense_split(const GemmArgs &a, int at, hipStream_t s);
// Sums the ks planes [ks][M][N] (fp32, in slice order) and applies the
// epilogue: EPI_RESID: C[p][n] = x[p][n] + gate[n] * sum (fp32), y[p][n] =
// sum when y != NULL; EPI_F32: C[p][n] = sum.  N a multiple of 4.
hipError_t launch_split_reduce(const float *planes, int ks, int64_t M, int64_t N, int epi, void *C,
                               const uint16_t *resid, const float *gate, float *y, hipStream_t s);

}  // namespace moe
