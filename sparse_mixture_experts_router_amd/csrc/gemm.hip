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
// Large-tile kernel (many rows per expert; dense projections at large T)
// ---------------------------------------------------------------------------
//
// Tile 256 (A rows) x 256 (B rows) x 32 (K) per stage, 256 threads as 2 x 2
// waves of 128 x 128, so a wave reads 16 KiB of LDS per stage for 64 MFMAs
// (64 FLOP per LDS byte).  Operands move global -> LDS with gfx950's
// direct-to-LDS loads (global_load_lds): a wave instruction fills LDS in lane
// order, so each lane fetches the global chunk that belongs at its LDS slot,
// which realises the XOR swizzle.  Four stage buffers rotate; the loads of
// K-tile kt+4 are issued at step kt, so three K-tiles (96 KiB per CU) are in
// flight while the MFMAs of one run.  Fragments are double-buffered in
// registers: the MFMAs on K-tile kt overlap the LDS reads of kt+1.
// When the MFMA type differs from the stored weights (bf16 weights with fp16
// activations, or MXFP4), each wave converts the share of the B stage that
// its own loads brought in, in LDS, two K-tiles ahead (bf16 -> fp16 in place;
// MXFP4 codes and block scales -> the activation type into the B operand
// area), so the MFMA operands always come straight from LDS reads.
// The MFMA operands are swapped (B first), so a lane's four accumulator
// elements are four consecutive output columns of one row: epilogue stores
// are 8 or 16 bytes wide.  EPI_SWIGLU tiles hold 128 gate rows then the 128
// matching up rows; wave column block c < 4 (gate) pairs with c + 4 (up).
// Rows past the tile's valid rows load a clamped valid A row; their results
// are never stored.  The half-height variant (HM) serves grouped tiles of at
// most 128 rows (an expert's remainder): its four waves share the 128 A rows
// and each takes 64 of the 256 B rows, so no wave idles on empty rows.

constexpr int kBigBM = kTileBM, kBigBN = kTileBN, kBigBK = 32;
static_assert(kBigBM == 256 && kBigBN == 256, "the wave layout below assumes 256x256 tiles");
constexpr int kBigOpBytes = kBigBM * kBigBK * 2;      // one operand area (A, or B in the MFMA type): 16 KiB
constexpr int kBigMxCodeBytes = kBigBN * kBigBK / 2;  // MXFP4 B codes per stage: 4 KiB
constexpr int kBigMxCodeOff = 2 * kBigOpBytes;        // MXFP4 codes, then 1 KiB of scale words
constexpr int kBigMxScaleOff = kBigMxCodeOff + kBigMxCodeBytes;
constexpr int kBigStageBytes = kBigMxScaleOff + kBigBN * 4;  // 37 KiB; 4 stages = 148 KiB

__shared__ __attribute__((aligned(16))) uint8_t big_lds0[kBigStageBytes];
__shared__ __attribute__((aligned(16))) uint8_t big_lds1[kBigStageBytes];
__shared__ __attribute__((aligned(16))) uint8_t big_lds2[kBigStageBytes];
__shared__ __attribute__((aligned(16))) uint8_t big_lds3[kBigStageBytes];

// Separate LDS objects per stage let the compiler see that a read of one
// stage does not depend on the loads still landing in the others.
template <int ST>
__device__ __forceinline__ uint8_t *big_buf() {
    if constexpr (ST == 0) return big_lds0;
    else if constexpr (ST == 1) return big_lds1;
    else if constexpr (ST == 2) return big_lds2;
    else return big_lds3;
}

#define MOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// 64-byte rows (32 x 16-bit): 16-byte chunk c of row r lives at chunk
// c ^ ((r >> 1) & 3), so the 8 rows a ds_read_b128 serves at once hit 8
// distinct 16-byte bank groups.
__device__ __forceinline__ int bswz(int row, int chunk) {
    return row * (kBigBK * 2) + ((chunk ^ ((row >> 1) & 3)) << 4);
}

// Load addresses: a wave-uniform base plus a 32-bit byte offset per lane, so
// the loads take the scalar-base form and the per-lane state stays small.
struct BigCtx {
    const uint8_t *A;       // activation base (uniform)
    uint32_t aoff[4];       // byte offsets of this lane's 4 A chunks at k = 0
    const uint8_t *B;       // first B row of the tile (bf16) or its code row (MXFP4) (uniform)
    uint32_t boff[4];       // bf16: byte offsets of this lane's 4 B chunks; MXFP4: [0] codes, [1] scales
    const uint8_t *bsc;     // MXFP4: scale base of the tile (uniform)
};

// Direct-to-LDS loads of K-tile kt into stage buffer ST.  A wave instruction
// fills 1 KiB of LDS in lane order (16 bytes per lane for dwordx4, 4 per lane
// for dword): 16 rows x 4 chunks of A or bf16 B, 64 rows x 16 bytes of MXFP4
// codes, or 64 rows' scale words.
template <int ST, bool MX, int HM>
__device__ __forceinline__ void big_issue(const BigCtx &c, int kt, int wave) {
    constexpr int NA = HM ? 2 : 4;  // A loads per wave (16 rows each)
    uint8_t *buf = big_buf<ST>();
    const uint8_t *Ak = c.A + (int64_t)kt * (kBigBK * 2);
#pragma unroll
    for (int i = 0; i < NA; ++i)
        __builtin_amdgcn_global_load_lds(Ak + c.aoff[i], MOE_LDS(buf + (wave * NA + i) * 1024), 16, 0, 0);
    if constexpr (MX) {
        __builtin_amdgcn_global_load_lds(c.B + (int64_t)kt * (kBigBK / 2) + c.boff[0],
                                         MOE_LDS(buf + kBigMxCodeOff + wave * 1024), 16, 0, 0);
        // the 4-byte-aligned word holding this K-tile's scale byte of the lane's row
        __builtin_amdgcn_global_load_lds(c.bsc + (int64_t)(kt & ~3) + c.boff[1],
                                         MOE_LDS(buf + kBigMxScaleOff + wave * 256), 4, 0, 0);
    } else {
        uint8_t *bb = buf + kBigOpBytes;
        const uint8_t *Bk = c.B + (int64_t)kt * (kBigBK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(Bk + c.boff[i], MOE_LDS(bb + (wave * 4 + i) * 1024), 16, 0, 0);
    }
}

template <bool MX, int AT> constexpr bool kBigConvert = MX || AT == ACT_F16;

// Convert the B data that this wave's own loads put into stage ST (K-tile kt)
// into the MFMA type: bf16 -> fp16 in place (the lane's own four chunks), or
// the 32 MXFP4 codes of row 64*wave + lane times its block scale -> four
// swizzled chunks of the B operand area.
template <int ST, bool MX, int AT>
__device__ __forceinline__ void big_convert(int kt, int wave, int lane) {
    uint8_t *buf = big_buf<ST>();
    uint8_t *bb = buf + kBigOpBytes;
    if constexpr (MX) {
        const int r = wave * 64 + lane;
        const uint4 codes = *(const uint4 *)(buf + kBigMxCodeOff + r * 16);
        const uint32_t sc = buf[kBigMxScaleOff + r * 4 + (kt & 3)];
        *(uint4 *)(bb + bswz(r, 0)) = mxfp4x8_to_act<AT>(codes.x, sc);
        *(uint4 *)(bb + bswz(r, 1)) = mxfp4x8_to_act<AT>(codes.y, sc);
        *(uint4 *)(bb + bswz(r, 2)) = mxfp4x8_to_act<AT>(codes.z, sc);
        *(uint4 *)(bb + bswz(r, 3)) = mxfp4x8_to_act<AT>(codes.w, sc);
    } else {
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = *(const uint4 *)(bb + (wave * 4 + i) * 1024 + lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) *(uint4 *)(bb + (wave * 4 + i) * 1024 + lane * 16) = bf16x8_to_f16x8(v[i]);
    }
}

// Fragments of one stage: A rows wm*128 + 16m + li, B rows bcol[c] + li, chunk lg.
template <int ST, int NBK>
__device__ __forceinline__ void big_read(uint4 (&fa)[8], uint4 (&fb)[NBK], const int (&bcol)[NBK], int wm, int li,
                                         int lg) {
    const uint8_t *buf = big_buf<ST>();
    const uint8_t *bb = buf + kBigOpBytes;
#pragma unroll
    for (int c = 0; c < NBK; ++c) fb[c] = *(const uint4 *)(bb + bswz(bcol[c] + li, lg));
#pragma unroll
    for (int m = 0; m < 8; ++m) fa[m] = *(const uint4 *)(buf + bswz(wm * 128 + m * 16 + li, lg));
}

template <int AT, int NBK>
__device__ __forceinline__ void big_mma(floatx4_t (&acc)[8][NBK], const uint4 (&fa)[8], const uint4 (&fb)[NBK]) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int c = 0; c < NBK; ++c) acc[m][c] = mfma16x16x32<AT>(fb[c], fa[m], acc[m][c]);
}

// Load instructions per wave per stage, and the vmcnt waits that leave 3 or
// 2 later stages in flight.  The waits go through the s_waitcnt builtin (not
// inline asm) so the compiler's own wait insertion knows of them.  gfx9
// s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);
template <bool MX, int HM> struct BigWait {
    static constexpr int kPerStage = (HM ? 2 : 4) + (MX ? 2 : 4);
    static __device__ __forceinline__ void keep3() { __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kPerStage)); }
    static __device__ __forceinline__ void keep2() { __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kPerStage)); }
    static __device__ __forceinline__ void all() { __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); }
};

// One K step j of a group of eight, on K-tile kt (stage ST = kt & 3).  On
// entry this wave holds the fragments of kt (cur) and has finished all its
// LDS work on earlier steps.  The barrier then guarantees for every wave that
// K-tile kt+1 is complete in its stage (landed, and converted where needed)
// and that nobody still reads stage ST, which receives K-tile kt+4 (clamped
// to the last K-tile near the end: those loads are never read).  The MFMAs on
// cur overlap the reads of kt+1 into nxt, except in the group's last step:
// fragments are not carried across the loop's back edge, which keeps the
// accumulators in place in the register allocation.  With conversion, the
// wave waits for its own loads of kt+2 and converts them halfway through the
// MFMAs, so the next barrier publishes kt+2 ready for use.
template <int J, bool MX, int AT, int HM, int NBK>
__device__ __forceinline__ void big_step(const BigCtx &c, floatx4_t (&acc)[8][NBK], const uint4 (&cur_a)[8],
                                         const uint4 (&cur_b)[NBK], uint4 (&nxt_a)[8], uint4 (&nxt_b)[NBK],
                                         const int (&bcol)[NBK], int kt, int nk, int wave, int wm, int lane) {
    constexpr int ST = J & 3;
    const int li = lane & 15, lg = lane >> 4;
    if constexpr (!kBigConvert<MX, AT>) BigWait<MX, HM>::keep2();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    big_issue<ST, MX, HM>(c, min(kt + 4, nk - 1), wave);
    if constexpr (J < 7) big_read<(ST + 1) & 3, NBK>(nxt_a, nxt_b, bcol, wm, li, lg);
    if constexpr (kBigConvert<MX, AT>) {
        // first half of the MFMAs (rows 0-3), then the conversion, then the rest
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int cc = 0; cc < NBK; ++cc) acc[m][cc] = mfma16x16x32<AT>(cur_b[cc], cur_a[m], acc[m][cc]);
        __builtin_amdgcn_sched_barrier(0);
        BigWait<MX, HM>::keep2();
        big_convert<(ST + 2) & 3, MX, AT>(kt + 2, wave, lane);
#pragma unroll
        for (int m = 4; m < 8; ++m)
#pragma unroll
            for (int cc = 0; cc < NBK; ++cc) acc[m][cc] = mfma16x16x32<AT>(cur_b[cc], cur_a[m], acc[m][cc]);
    } else {
        big_mma<AT, NBK>(acc, cur_a, cur_b);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
}

template <int EPI, bool MX, bool GROUPED, int AT, int OT, int HM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_big_kernel(GemmArgs a) {
    constexpr int NBK = HM ? 4 : 8;      // 16-column blocks per wave
    constexpr int NA = HM ? 2 : 4;       // A loads per wave per stage
    constexpr int BM = HM ? kHalfBM : kBigBM;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = HM ? 0 : wave >> 1, wn = HM ? wave : wave & 1;
    const int li = lane & 15, lg = lane >> 4;
    constexpr int WCOLS = HM ? 64 : 128;  // output-space B rows per wave (SWIGLU: half gate, half up)

    const int64_t K = a.K;
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / (kBigBN / 2) : a.N / kBigBN;
    const int ntiles = GROUPED ? *a.ntiles : (int)((a.M + BM - 1) / BM);
    const int64_t items = (int64_t)ntiles * nblocks;
    const int nk = (int)(K / kBigBK);  // a multiple of 8
    // Direct-load lane mapping of 64-byte rows: lane l fills row 16q + (l >> 2),
    // physical chunk l & 3, i.e. logical chunk (l & 3) ^ ((l >> 3) & 3).
    const int drow = lane >> 2, dchunk = (lane & 3) ^ ((lane >> 3) & 3);

    int bcol[NBK];
#pragma unroll
    for (int c = 0; c < NBK; ++c) {
        if constexpr (EPI == EPI_SWIGLU)
            bcol[c] = (c < NBK / 2) ? wn * (WCOLS / 2) + c * 16 : 128 + wn * (WCOLS / 2) + (c - NBK / 2) * 16;
        else
            bcol[c] = wn * WCOLS + c * 16;
    }

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        // Tile-major order: the column blocks of one row tile run side by side
        // (its A rows stay in L2) and so do the row tiles of one expert.
        const int t = (int)(item / nblocks);
        const int64_t nb = item - (int64_t)t * nblocks;
        RowTile rt;
        load_tile(a, GROUPED, BM, t, rt);
        const int64_t brow0 = GROUPED ? (int64_t)rt.e * a.b_group_rows : 0;

        BigCtx c;
        c.A = (const uint8_t *)a.A;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int row = min(wave * (NA * 16) + i * 16 + drow, rt.mcount - 1);
            const int64_t p = rt.p0 + row;
            const int64_t arow = a.a_gather ? (int64_t)a.a_gather[p] : p;
            c.aoff[i] = (uint32_t)((arow * a.lda + dchunk * 8) * 2);
        }
        // The tile's B rows 0..255: SWIGLU rows 0-127 are gate rows nb*128.., rows
        // 128-255 the matching up rows N + nb*128..; a lane loads tile rows
        // 64*wave + 16i + drow (bf16) or 64*wave + lane (MXFP4).
        const int64_t bfirst = brow0 + ((EPI == EPI_SWIGLU) ? nb * 128 : nb * kBigBN);
        const int64_t upskip = (EPI == EPI_SWIGLU) ? a.N - 128 : 0;  // rows 128.. sit this far further on
        auto brel = [&](int row) -> int64_t { return row + (row >= 128 ? upskip : 0); };
        if constexpr (MX) {
            const int row = wave * 64 + lane;
            c.B = (const uint8_t *)a.B + bfirst * (K / 2);
            c.bsc = (const uint8_t *)a.B + a.b_rows_total * (K / 2) + bfirst * (K / 32);
            c.boff[0] = (uint32_t)(brel(row) * (K / 2));
            c.boff[1] = (uint32_t)(brel(row) * (K / 32));
            c.boff[2] = c.boff[3] = 0;
        } else {
            c.B = (const uint8_t *)((const uint16_t *)a.B + bfirst * K);
#pragma unroll
            for (int i = 0; i < 4; ++i) c.boff[i] = (uint32_t)((brel(wave * 64 + i * 16 + drow) * K + dchunk * 8) * 2);
            c.bsc = nullptr;
        }

        floatx4_t acc[8][NBK];
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int cc = 0; cc < NBK; ++cc) acc[m][cc] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        big_issue<0, MX, HM>(c, 0, wave);
        big_issue<1, MX, HM>(c, 1, wave);
        big_issue<2, MX, HM>(c, 2, wave);
        big_issue<3, MX, HM>(c, 3, wave);
        if constexpr (kBigConvert<MX, AT>) {
            BigWait<MX, HM>::keep2();
            big_convert<0, MX, AT>(0, wave, lane);
            big_convert<1, MX, AT>(1, wave, lane);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        } else {
            BigWait<MX, HM>::keep3();
        }
        __builtin_amdgcn_s_barrier();
        for (int kt = 0; kt < nk; kt += 8) {
            // K-tile kt is complete for every wave (barrier above or step 7 below).
            uint4 fa0[8], fb0[NBK], fa1[8], fb1[NBK];
            big_read<0, NBK>(fa0, fb0, bcol, wm, li, lg);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            big_step<0, MX, AT, HM, NBK>(c, acc, fa0, fb0, fa1, fb1, bcol, kt + 0, nk, wave, wm, lane);
            big_step<1, MX, AT, HM, NBK>(c, acc, fa1, fb1, fa0, fb0, bcol, kt + 1, nk, wave, wm, lane);
            big_step<2, MX, AT, HM, NBK>(c, acc, fa0, fb0, fa1, fb1, bcol, kt + 2, nk, wave, wm, lane);
            big_step<3, MX, AT, HM, NBK>(c, acc, fa1, fb1, fa0, fb0, bcol, kt + 3, nk, wave, wm, lane);
            big_step<4, MX, AT, HM, NBK>(c, acc, fa0, fb0, fa1, fb1, bcol, kt + 4, nk, wave, wm, lane);
            big_step<5, MX, AT, HM, NBK>(c, acc, fa1, fb1, fa0, fb0, bcol, kt + 5, nk, wave, wm, lane);
            big_step<6, MX, AT, HM, NBK>(c, acc, fa0, fb0, fa1, fb1, bcol, kt + 6, nk, wave, wm, lane);
            big_step<7, MX, AT, HM, NBK>(c, acc, fa1, fb1, fa0, fb0, bcol, kt + 7, nk, wave, wm, lane);
        }
        // Drain the clamped tail loads before the stages are refilled.
        BigWait<MX, HM>::all();
        __builtin_amdgcn_s_barrier();

        // Epilogue: lane (li, lg) holds row wm*128 + 16m + li, columns
        // bcol[c] + 4lg + q (q = 0..3) of every block.
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int row = wm * 128 + m * 16 + li;
            const bool ok = row < rt.mcount;
            const int64_t p = rt.p0 + row;
            if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int cc = 0; cc < NBK / 2; ++cc) {
                    if (ok) {
                        uint16_t h[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            h[q] = f32_to_act<OT>(silu(acc[m][cc][q]) * acc[m][cc + NBK / 2][q]);
                        const int64_t j = nb * 128 + wn * (WCOLS / 2) + cc * 16 + lg * 4;
                        *(uint2 *)((uint16_t *)a.C + p * a.ldc + j) =
                            make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                    }
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < NBK; ++cc) {
                    const int64_t n = nb * kBigBN + wn * WCOLS + cc * 16 + lg * 4;
                    const floatx4_t v = acc[m][cc];
                    if constexpr (EPI == EPI_F32) {
                        if (ok) *(floatx4_t *)((float *)a.C + p * a.ldc + n) = v;
                    } else if constexpr (EPI == EPI_ACT) {
                        if (ok)
                            *(uint2 *)((uint16_t *)a.C + p * a.ldc + n) =
                                make_uint2(f32_to_act<OT>(v[0]) | ((uint32_t)f32_to_act<OT>(v[1]) << 16),
                                           f32_to_act<OT>(v[2]) | ((uint32_t)f32_to_act<OT>(v[3]) << 16));
                    } else if constexpr (EPI == EPI_NORM) {
                        uint16_t h[4];
                        float sq = 0.f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float gsc = a.gamma ? 1.0f + a.gamma[n + q] : 1.0f;
                            h[q] = f32_to_bf16(gsc * v[q]);
                            const float e = a.norm_round ? bf16_to_f32(h[q]) : v[q];
                            sq += e * e;
                        }
                        if (ok)
                            *(uint2 *)((uint16_t *)a.C + p * a.ldc + n) =
                                make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                        sq += __shfl_xor(sq, 16, 64);
                        sq += __shfl_xor(sq, 32, 64);
                        if (ok && lg == 0) a.ssq[p * a.nparts + nb * 16 + wn * (WCOLS / 16) + cc] = sq;
                    } else {  // EPI_RESID
                        if (ok) {
                            const uint2 hx = *(const uint2 *)(a.resid + p * a.N + n);
                            const float4 g = *(const float4 *)(a.gate + n);
                            floatx4_t o;
                            o[0] = bf16_to_f32((uint16_t)hx.x) + g.x * v[0];
                            o[1] = bf16_to_f32((uint16_t)(hx.x >> 16)) + g.y * v[1];
                            o[2] = bf16_to_f32((uint16_t)hx.y) + g.z * v[2];
                            o[3] = bf16_to_f32((uint16_t)(hx.y >> 16)) + g.w * v[3];
                            *(floatx4_t *)((float *)a.C + p * a.ldc + n) = o;
                            if (a.y) *(floatx4_t *)(a.y + p * a.N + n) = v;
                        }
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
constexpr int kBigGrid = 256;      // persistent grid cap of the large-tile kernel (one per CU)

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

template <int EPI, bool MX, bool GROUPED, int AT, int OT, int HM>
static hipError_t run_tile(const GemmArgs &a, hipStream_t s) {
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / (kBigBN / 2) : a.N / kBigBN;
    const int64_t tiles = GROUPED ? a.max_tiles : (a.M + kBigBM - 1) / kBigBM;
    const int64_t items = tiles * nblocks;
    if (items <= 0) return hipSuccess;
    const int grid = (int)(items < kBigGrid ? items : kBigGrid);
    gemm_big_kernel<EPI, MX, GROUPED, AT, OT, HM><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

// Dense launches use 64-row tiles on the streaming kernel, grouped ones 16-row tiles.
template <int EPI, int NB, bool MX, bool GROUPED, int AT, int OT>
static hipError_t run_path(const GemmArgs &a, int path, hipStream_t s) {
    if (path == PATH_TILE) return run_tile<EPI, MX, GROUPED, AT, OT, 0>(a, s);
    if (path == PATH_HALF) {
        if constexpr (GROUPED) return run_tile<EPI, MX, GROUPED, AT, OT, 1>(a, s);
        else return hipErrorInvalidValue;
    }
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
