// Arguments and launchers of the layer's MFMA GEMMs: C = A * B^T with A rows
// of bf16 activations and B rows of bf16 or MXFP4 weights (both with the
// reduction dimension K contiguous), fp32 accumulation, fused epilogues.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum Epi : int {
    EPI_F32 = 0,     // C[p][n] = acc (fp32)
    EPI_BF16 = 1,    // C[p][n] = bf16(acc)
    EPI_SWIGLU = 2,  // C[p][j] = bf16(silu(acc[j]) * acc[F + j]); B holds gate rows then up rows
    EPI_NORM = 3,    // C[p][n] = s = bf16((1 + gamma[n]) * acc); ssq[p][nb] = sum over the block of s^2
    EPI_RESID = 4    // out[p][n] = x[p][n] + gate[n] * acc (fp32); y[p][n] = acc when y != NULL
};

struct TileEntry {  // one M-tile of a grouped GEMM: expert e, rows m0 .. of its segment
    int32_t e;
    int32_t m0;
};

struct GemmArgs {
    // A: bf16 rows with leading dimension lda.  Grouped GEMMs index rows by
    // permuted position p; a_gather (may be NULL) maps p to the A row.
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
    int32_t norm_round;    // EPI_NORM: 1 rounds the scaled vector to bf16 before squaring
    const uint16_t *resid; // EPI_RESID: x rows (bf16), leading dimension N
    const float *gate;     // EPI_RESID: g [N]
    float *y;              // EPI_RESID: optional y [rows][N]
};

// Columns of output that one work item of each kernel covers.
constexpr int kStreamCols = 16;   // per 16-column block; SWIGLU items cover 16 outputs (32 B rows)
constexpr int kTileBM = 128;
constexpr int kTileBN = 128;      // B rows per tile (SWIGLU: 64 gate + 64 up -> 64 outputs)
constexpr int kTileBK = 64;
constexpr int kSmallBM = 16;      // rows per tile of the streaming kernel's grouped lists

// Launchers (return hipError_t of the launch).
// Streaming kernel: weights streamed straight into MFMA registers, K split
// over the 4 waves of a workgroup.  mb: 16-row blocks per tile (1..4).
hipError_t launch_gemm_stream(const GemmArgs &a, int epi, bool mx, bool grouped, int mb, int grid_cap,
                              hipStream_t s);
// LDS-tiled kernel: 128x128x64 tiles, double-buffered LDS, 4 waves of 64x64.
hipError_t launch_gemm_tile(const GemmArgs &a, int epi, bool mx, bool grouped, int grid_cap, hipStream_t s);

}  // namespace moe
