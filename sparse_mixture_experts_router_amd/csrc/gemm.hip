// MFMA GEMMs of the latent MoE layer for gfx950 (CDNA4).
//
// Both kernels compute C = A * B^T with bf16 A rows (activations), bf16 or
// MXFP4 B rows (weights), fp32 accumulation on v_mfma_f32_16x16x32_bf16, and
// one of the fused epilogues of gemm.h.  Grouped launches walk a device-side
// list of (expert, first row) tiles built by the permutation kernel, so the
// host never waits for the routing result; the grid is persistent and reads
// the list length from device memory.
//
// Sources of the arithmetic (page titles and sections):
//  - expert shapes, SwiGLU, gate/up packing and the latent projections:
//    flozi.net "Muse Spark Open: Norm-Preserving Gates Are Not a Norm
//    Guarantee", section "Latent experts: normalization happens before the
//    weighted sum"; no GLU clamp or FFN bias: archdb "Muse-Spark-Open-816B-A42B";
//  - per-expert input-scaled norm (scaled vector rounded to the input dtype
//    before an FP32 reduction): same page, sections "Two normalization orders
//    implement different functions" and "Latent experts ...";
//  - the weight-bandwidth-bound small-batch regime each expert sees:
//    bobbyburns.tech "816 billion parameters, and only 42 billion show up for
//    each token", section "Connecting the dots".
#include "common.h"
#include "gemm.h"

namespace moe {

// ---------------------------------------------------------------------------
// Shared epilogue pieces
// ---------------------------------------------------------------------------

struct RowTile {
    int64_t p0;     // first output row (permuted position or token)
    int32_t e;      // expert (0 when dense)
    int32_t mcount; // valid rows in this tile
};

__device__ __forceinline__ bool load_tile(const GemmArgs &a, bool grouped, int bm, int t, RowTile &rt) {
    if (grouped) {
        TileEntry te = a.tiles[t];
        int c = a.counts[te.e];
        rt.e = te.e;
        rt.p0 = (int64_t)a.offsets[te.e] + te.m0;
        rt.mcount = min(bm, c - te.m0);
    } else {
        rt.e = 0;
        rt.p0 = (int64_t)t * bm;
        rt.mcount = (int)min<int64_t>(bm, a.M - rt.p0);
    }
    return rt.mcount > 0;
}

// Store one accumulator element of a non-SwiGLU epilogue.  Returns the value
// whose square feeds the norm's partial sum (EPI_NORM), else 0.
template <int EPI, int OT>
__device__ __forceinline__ float store_elem(const GemmArgs &a, int64_t p, int64_t n, float v) {
    if constexpr (EPI == EPI_F32) {
        ((float *)a.C)[p * a.ldc + n] = v;
        return 0.f;
    } else if constexpr (EPI == EPI_ACT) {
        ((uint16_t *)a.C)[p * a.ldc + n] = f32_to_act<OT>(v);
        return 0.f;
    } else if constexpr (EPI == EPI_NORM) {
        float gsc = a.gamma ? 1.0f + a.gamma[n] : 1.0f;
        uint16_t s = f32_to_bf16(gsc * v);
        ((uint16_t *)a.C)[p * a.ldc + n] = s;
        float q = a.norm_round ? bf16_to_f32(s) : v;
        return q * q;
    } else {  // EPI_RESID
        float h = bf16_to_f32(a.resid[p * a.N + n]);
        ((float *)a.C)[p * a.ldc + n] = h + a.gate[n] * v;
        if (a.y) a.y[p * a.N + n] = v;
        return 0.f;
    }
}

// Sum over the 16 lanes that share l/16 (one output row per element index).
__device__ __forceinline__ float sum16(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Streaming kernel (small row counts per expert: weight-bandwidth bound)
// ---------------------------------------------------------------------------
//
// Work item = (row tile, column block).  A column block is NB blocks of 16 B
// rows (EPI_SWIGLU: NB = 2, the gate rows j0.. and the up rows F + j0..).
// The 4 waves of the workgroup split K in four contiguous quarters.  Every
// 128-wide K group is one lane-group-permuted MFMA quartet: lane group
// g = lane/16 owns k in [32g, 32g+32) of the group and feeds 8 of them to
// each of 4 MFMAs, so a lane reads 64 contiguous bytes of a bf16 B row (or
// one whole 32-element MXFP4 block: 16 code bytes and its scale) and the
// same 64 bytes of its A row.  Partial sums of the waves meet in LDS and
// wave 0 applies the epilogue.

template <int MB, int NB>
struct StreamFrag {
    uint4 b[NB][4];
    uint4 a[MB][4];
};

template <int MB, int NB, bool MX, int AT>
__device__ __forceinline__ void stream_load(StreamFrag<MB, NB> &f, const uint8_t *const bptr[NB],
                                            const uint8_t *const bscale[NB], const uint16_t *const aptr[MB],
                                            int64_t kk) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        if constexpr (MX) {
            uint4 codes = *(const uint4 *)(bptr[c] + (kk >> 1));
            uint32_t sc = bscale[c][kk >> 5];
            f.b[c][0] = mxfp4x8_to_act<AT>(codes.x, sc);
            f.b[c][1] = mxfp4x8_to_act<AT>(codes.y, sc);
            f.b[c][2] = mxfp4x8_to_act<AT>(codes.z, sc);
            f.b[c][3] = mxfp4x8_to_act<AT>(codes.w, sc);
        } else {
            const uint4 *p = (const uint4 *)(bptr[c] + kk * 2);
#pragma unroll
            for (int s = 0; s < 4; ++s) f.b[c][s] = weight_bf16_as<AT>(p[s]);
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        if (aptr[m]) {
            const uint4 *p = (const uint4 *)(aptr[m] + kk);
#pragma unroll
            for (int s = 0; s < 4; ++s) f.a[m][s] = p[s];
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) f.a[m][s] = make_uint4(0, 0, 0, 0);
        }
    }
}

template <int MB, int NB, int EPI, bool MX, bool GROUPED, int AT, int OT>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs a) {
    constexpr int BM = 16 * MB;
    __shared__ floatx4_t red[3][MB][NB][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;  // row (A) / column (B) within a 16-block
    const int lg = lane >> 4;  // k group of 32 within a 128-wide K group

    const int64_t K = a.K;
    const int64_t kq = K / 4;            // K range of one wave
    const int64_t kbeg = wave * kq;
    const int64_t kend = kbeg + kq;
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / 16 : a.N / (16 * NB);
    const int ntiles = GROUPED ? *a.ntiles : (int)((a.M + BM - 1) / BM);
    const int64_t items = (int64_t)ntiles * nblocks;

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int t = (int)(item / nblocks);
        const int64_t nb = item - (int64_t)t * nblocks;
        RowTile rt;
        load_tile(a, GROUPED, BM, t, rt);  // mcount > 0 for every listed tile

        // B row pointers (lane's row li of each 16-row block) and A row pointers.
        const uint8_t *bptr[NB];
        const uint8_t *bscale[NB];
        int64_t brow0 = GROUPED ? (int64_t)rt.e * a.b_group_rows : 0;
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            int64_t r;
            if constexpr (EPI == EPI_SWIGLU)
                r = brow0 + (c == 0 ? 0 : a.N) + nb * 16 + li;
            else
                r = brow0 + (nb * NB + c) * 16 + li;
            if constexpr (MX) {
                // lane group lg reads its 32-element block of each 128-wide group
                bptr[c] = (const uint8_t *)a.B + r * (K / 2) + (lg * 32) / 2;
                bscale[c] = (const uint8_t *)a.B + a.b_rows_total * (K / 2) + r * (K / 32) + lg;
            } else {
                bptr[c] = (const uint8_t *)a.B + (r * K + lg * 32) * 2;
                bscale[c] = nullptr;
            }
        }
        const uint16_t *aptr[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            int row = m * 16 + li;
            if (row < rt.mcount) {
                int64_t p = rt.p0 + row;
                int64_t arow = a.a_gather ? (int64_t)a.a_gather[p] : p;
                aptr[m] = a.A + arow * a.lda + lg * 32;
            } else {
                aptr[m] = nullptr;
            }
        }

        floatx4_t acc[MB][NB];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int c = 0; c < NB; ++c) acc[m][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        StreamFrag<MB, NB> cur, nxt;
        stream_load<MB, NB, MX, AT>(cur, bptr, bscale, aptr, kbeg);
        for (int64_t kk = kbeg; kk < kend; kk += 128) {
            if (kk + 128 < kend) stream_load<MB, NB, MX, AT>(nxt, bptr, bscale, aptr, kk + 128);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int c = 0; c < NB; ++c)
                        acc[m][c] = mfma16x16x32<AT>(cur.a[m][s], cur.b[c][s], acc[m][c]);
            cur = nxt;
        }

        // Cross-wave reduction, fixed order: wave0 + wave1 + wave2 + wave3.
        if (wave > 0) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int c = 0; c < NB; ++c) red[wave - 1][m][c][lane] = acc[m][c];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 0; w < 3; ++w)
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int c = 0; c < NB; ++c) acc[m][c] += red[w][m][c][lane];

            // Epilogue: lane holds rows 4*lg + q (q = 0..3) of each row block, column li.
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                float rowsq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int row = m * 16 + lg * 4 + q;
                    bool ok = row < rt.mcount;
                    int64_t p = rt.p0 + row;
                    if constexpr (EPI == EPI_SWIGLU) {
                        if (ok) {
                            float g = acc[m][0][q], u = acc[m][NB - 1][q];
                            ((uint16_t *)a.C)[p * a.ldc + nb * 16 + li] = f32_to_act<OT>(silu(g) * u);
                        }
                    } else {
#pragma unroll
                        for (int c = 0; c < NB; ++c) {
                            int64_t n = (nb * NB + c) * 16 + li;
                            if (ok) rowsq[q] += store_elem<EPI, OT>(a, p, n, acc[m][c][q]);
                        }
                    }
                }
                if constexpr (EPI == EPI_NORM) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = sum16(rowsq[q]);
                        int row = m * 16 + lg * 4 + q;
                        if (li == 0 && row < rt.mcount) a.ssq[(rt.p0 + row) * a.nparts + nb] = v;
                    }
                }
            }
        }
        __syncthreads();  // red[] is reused by the next item
    }
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel (many rows per expert: MFMA bound)
// ---------------------------------------------------------------------------
//
// Tile 128 (rows of A) x 128 (rows of B) x 64 (K), 256 threads as 2 x 2
// waves of 64 x 64.  Each stage holds A and B as [128][64] bf16 with the
// 16-byte chunk index XOR-swizzled by (row & 7), double-buffered; the next
// stage is fetched into registers while the current one is multiplied.
// EPI_SWIGLU tiles hold 64 gate rows then the 64 matching up rows, and each
// wave's four column blocks are two gate blocks and their two up blocks.

constexpr int kLdsTile = kTileBM * kTileBK;  // bf16 elements per operand stage

__device__ __forceinline__ int swz(int row, int chunk) { return row * kTileBK + ((chunk ^ (row & 7)) << 3); }

template <int EPI, bool MX, bool GROUPED, int AT, int OT>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kLdsTile];  // [stage][A/B]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 15, lg = lane >> 4;

    const int64_t K = a.K;
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / 64 : a.N / kTileBN;
    const int ntiles = GROUPED ? *a.ntiles : (int)((a.M + kTileBM - 1) / kTileBM);
    const int64_t items = (int64_t)ntiles * nblocks;
    const int nk = (int)(K / kTileBK);

    // Global->LDS assignment: bf16 operands: thread loads rows (tid>>3) + 32r, chunk tid&7.
    const int lrow = tid >> 3, lchunk = tid & 7;
    // MXFP4 B: thread handles row tid>>1, 32-element half (tid&1).
    const int mrow = tid >> 1, mhalf = tid & 1;

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int t = (int)(item % ntiles);
        const int64_t nb = item / ntiles;
        RowTile rt;
        load_tile(a, GROUPED, kTileBM, t, rt);
        const int64_t brow0 = GROUPED ? (int64_t)rt.e * a.b_group_rows : 0;

        // A source rows for this thread's 4 load slots.
        const uint16_t *asrc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int row = lrow + 32 * r;
            if (row < rt.mcount) {
                int64_t p = rt.p0 + row;
                int64_t arow = a.a_gather ? (int64_t)a.a_gather[p] : p;
                asrc[r] = a.A + arow * a.lda + lchunk * 8;
            } else {
                asrc[r] = nullptr;
            }
        }
        // B source rows.
        auto brow_of = [&](int row) -> int64_t {
            if constexpr (EPI == EPI_SWIGLU)
                return brow0 + (row < 64 ? nb * 64 + row : a.N + nb * 64 + (row - 64));
            else
                return brow0 + nb * kTileBN + row;
        };
        const uint16_t *bsrc[4];
        const uint8_t *bcode = nullptr, *bsc = nullptr;
        if constexpr (MX) {
            int64_t r = brow_of(mrow);
            bcode = (const uint8_t *)a.B + r * (K / 2) + mhalf * 16;
            bsc = (const uint8_t *)a.B + a.b_rows_total * (K / 2) + r * (K / 32) + mhalf;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) bsrc[r] = (const uint16_t *)a.B + brow_of(lrow + 32 * r) * K + lchunk * 8;
        }

        uint4 ra[4], rb[4];
        auto gload = [&](int kt) {
            int64_t k0 = (int64_t)kt * kTileBK;
#pragma unroll
            for (int r = 0; r < 4; ++r) ra[r] = asrc[r] ? *(const uint4 *)(asrc[r] + k0) : make_uint4(0, 0, 0, 0);
            if constexpr (MX) {
                uint4 codes = *(const uint4 *)(bcode + k0 / 2);
                uint32_t sc = bsc[k0 / 32];
                rb[0] = mxfp4x8_to_act<AT>(codes.x, sc);
                rb[1] = mxfp4x8_to_act<AT>(codes.y, sc);
                rb[2] = mxfp4x8_to_act<AT>(codes.z, sc);
                rb[3] = mxfp4x8_to_act<AT>(codes.w, sc);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) rb[r] = *(const uint4 *)(bsrc[r] + k0);
            }
        };
        auto lstore = [&](int st) {
            uint16_t *la = lds[st][0], *lb = lds[st][1];
#pragma unroll
            for (int r = 0; r < 4; ++r) *(uint4 *)(la + swz(lrow + 32 * r, lchunk)) = ra[r];
            if constexpr (MX) {
#pragma unroll
                for (int c = 0; c < 4; ++c) *(uint4 *)(lb + swz(mrow, mhalf * 4 + c)) = rb[c];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) *(uint4 *)(lb + swz(lrow + 32 * r, lchunk)) = rb[r];
            }
        };

        // Wave's B-tile rows of its 4 column blocks.
        int bcol[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (EPI == EPI_SWIGLU)
                bcol[c] = (c < 2) ? wn * 32 + c * 16 : 64 + wn * 32 + (c - 2) * 16;
            else
                bcol[c] = wn * 64 + c * 16;
        }

        floatx4_t acc[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[m][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        gload(0);
        if constexpr (!MX && AT == ACT_F16) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rb[r] = bf16x8_to_f16x8(rb[r]);
        }
        lstore(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            if (kt + 1 < nk) gload(kt + 1);
            const uint16_t *la = lds[st][0], *lb = lds[st][1];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                uint4 fa[4], fb[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) fa[m] = *(const uint4 *)(la + swz(wm * 64 + m * 16 + li, s * 4 + lg));
#pragma unroll
                for (int c = 0; c < 4; ++c) fb[c] = *(const uint4 *)(lb + swz(bcol[c] + li, s * 4 + lg));
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[m][c] = mfma16x16x32<AT>(fa[m], fb[c], acc[m][c]);
            }
            if (kt + 1 < nk) {
                if constexpr (!MX && AT == ACT_F16) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) rb[r] = bf16x8_to_f16x8(rb[r]);
                }
                lstore(st ^ 1);
            }
            __syncthreads();
        }

        // Epilogue.  EPI_NORM partial sums are per 16-column block, the same
        // layout the streaming kernel writes (nparts = N / 16 per row).
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int row = wm * 64 + m * 16 + lg * 4 + q;
                bool ok = row < rt.mcount;
                int64_t p = rt.p0 + row;
                if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        if (ok) {
                            float g = acc[m][c][q], u = acc[m][c + 2][q];
                            int64_t j = nb * 64 + wn * 32 + c * 16 + li;
                            ((uint16_t *)a.C)[p * a.ldc + j] = f32_to_act<OT>(silu(g) * u);
                        }
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        int64_t n = nb * kTileBN + wn * 64 + c * 16 + li;
                        float sq = ok ? store_elem<EPI, OT>(a, p, n, acc[m][c][q]) : 0.f;
                        if constexpr (EPI == EPI_NORM) {
                            sq = sum16(sq);
                            if (li == 0 && ok) a.ssq[p * a.nparts + nb * 8 + wn * 4 + c] = sq;
                        }
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

constexpr int kStreamGrid = 4096;  // persistent grid cap of the streaming kernel
constexpr int kTileGrid = 512;     // persistent grid cap of the tiled kernel

template <int MB, int NB, int EPI, bool MX, bool GROUPED, int AT, int OT>
static hipError_t run_stream(const GemmArgs &a, hipStream_t s) {
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / 16 : a.N / (16 * NB);
    const int64_t tiles = GROUPED ? a.max_tiles : (a.M + 16 * MB - 1) / (16 * MB);
    const int64_t items = tiles * nblocks;
    if (items <= 0) return hipSuccess;
    const int grid = (int)(items < kStreamGrid ? items : kStreamGrid);
    gemm_stream_kernel<MB, NB, EPI, MX, GROUPED, AT, OT><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int EPI, bool MX, bool GROUPED, int AT, int OT>
static hipError_t run_tile(const GemmArgs &a, hipStream_t s) {
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / 64 : a.N / kTileBN;
    const int64_t tiles = GROUPED ? a.max_tiles : (a.M + kTileBM - 1) / kTileBM;
    const int64_t items = tiles * nblocks;
    if (items <= 0) return hipSuccess;
    const int grid = (int)(items < kTileGrid ? items : kTileGrid);
    gemm_tile_kernel<EPI, MX, GROUPED, AT, OT><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

// Dense launches use 64-row tiles on the streaming kernel, grouped ones 16-row tiles.
template <int EPI, int NB, bool MX, bool GROUPED, int AT, int OT>
static hipError_t run_path(const GemmArgs &a, int path, hipStream_t s) {
    if (path == PATH_TILE) return run_tile<EPI, MX, GROUPED, AT, OT>(a, s);
    if constexpr (GROUPED) return run_stream<1, NB, EPI, MX, GROUPED, AT, OT>(a, s);
    else return run_stream<4, NB, EPI, MX, GROUPED, AT, OT>(a, s);
}

hipError_t launch_router_gemm(const GemmArgs &a, int path, hipStream_t s) {
    return run_path<EPI_F32, 1, false, false, ACT_BF16, ACT_BF16>(a, path, s);
}

hipError_t launch_down_gemm(const GemmArgs &a, int path, bool mx, int ot, hipStream_t s) {
    if (mx) {
        if (ot == ACT_F16) return run_path<EPI_ACT, 1, true, false, ACT_BF16, ACT_F16>(a, path, s);
        return run_path<EPI_ACT, 1, true, false, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (ot == ACT_F16) return run_path<EPI_ACT, 1, false, false, ACT_BF16, ACT_F16>(a, path, s);
    return run_path<EPI_ACT, 1, false, false, ACT_BF16, ACT_BF16>(a, path, s);
}

hipError_t launch_gemm1(const GemmArgs &a, int path, bool mx, int at, hipStream_t s) {
    if (mx) {
        if (at == ACT_F16) return run_path<EPI_SWIGLU, 2, true, true, ACT_F16, ACT_F16>(a, path, s);
        return run_path<EPI_SWIGLU, 2, true, true, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (at == ACT_F16) return run_path<EPI_SWIGLU, 2, false, true, ACT_F16, ACT_F16>(a, path, s);
    return run_path<EPI_SWIGLU, 2, false, true, ACT_BF16, ACT_BF16>(a, path, s);
}

hipError_t launch_gemm2(const GemmArgs &a, int path, bool mx, int at, bool norm, hipStream_t s) {
    if (norm) {
        if (mx) {
            if (at == ACT_F16) return run_path<EPI_NORM, 1, true, true, ACT_F16, ACT_BF16>(a, path, s);
            return run_path<EPI_NORM, 1, true, true, ACT_BF16, ACT_BF16>(a, path, s);
        }
        if (at == ACT_F16) return run_path<EPI_NORM, 1, false, true, ACT_F16, ACT_BF16>(a, path, s);
        return run_path<EPI_NORM, 1, false, true, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (mx) {
        if (at == ACT_F16) return run_path<EPI_ACT, 1, true, true, ACT_F16, ACT_BF16>(a, path, s);
        return run_path<EPI_ACT, 1, true, true, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (at == ACT_F16) return run_path<EPI_ACT, 1, false, true, ACT_F16, ACT_BF16>(a, path, s);
    return run_path<EPI_ACT, 1, false, true, ACT_BF16, ACT_BF16>(a, path, s);
}

hipError_t launch_up_gemm(const GemmArgs &a, int path, bool mx, int at, bool resid, hipStream_t s) {
    if (resid) {
        if (mx) {
            if (at == ACT_F16) return run_path<EPI_RESID, 1, true, false, ACT_F16, ACT_BF16>(a, path, s);
            return run_path<EPI_RESID, 1, true, false, ACT_BF16, ACT_BF16>(a, path, s);
        }
        if (at == ACT_F16) return run_path<EPI_RESID, 1, false, false, ACT_F16, ACT_BF16>(a, path, s);
        return run_path<EPI_RESID, 1, false, false, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (mx) {
        if (at == ACT_F16) return run_path<EPI_F32, 1, true, false, ACT_F16, ACT_BF16>(a, path, s);
        return run_path<EPI_F32, 1, true, false, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (at == ACT_F16) return run_path<EPI_F32, 1, false, false, ACT_F16, ACT_BF16>(a, path, s);
    return run_path<EPI_F32, 1, false, false, ACT_BF16, ACT_BF16>(a, path, s);
}

}  // namespace moe
