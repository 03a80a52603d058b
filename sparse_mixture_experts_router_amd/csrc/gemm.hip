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
        const TileEntry te = a.tiles[t];  // rows and count precomputed with the list
        rt.e = te.e;
        rt.p0 = te.p0;
        rt.mcount = te.mcount;
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

#define MOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Cache policy of the weight loads: every weight block is read once, and
// the non-temporal (nt) policy moves them measurably faster (7.0 vs 6.2 TB/s
// for a pure weight stream on this chip).
constexpr int kStreamPolicy = 2;  // nt

// Waits go through the s_waitcnt builtin (not inline asm) so the compiler's
// own wait insertion knows of them.  gfx9 s_waitcnt fields: vmcnt bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// ---------------------------------------------------------------------------
// Streaming kernel (small row counts per expert: weight-bandwidth bound)
// ---------------------------------------------------------------------------
//
// Work item = (row tile, column block).  A column block is NB blocks of 16 B
// rows (EPI_SWIGLU: NB / 2 gate blocks of rows j0.. and the matching up
// blocks of rows F + j0..).  The 4 waves of the workgroup split K between
// them.  Items on bf16/fp16 weights (grouped 16-row and dense 64-row tiles)
// stage A and B through LDS (below).  Items on MXFP4 weights load straight
// into registers: every 128-wide K group is one lane-group-permuted MFMA
// quartet, lane group g = lane/16 owning k in [32g, 32g+32) of the group and
// feeding 8 of them to each of 4 MFMAs, so a lane reads one whole 32-element
// MXFP4 block (16 code bytes; its scale comes from scale words, below) and
// the same 64 bytes of its A row.  Grouped MXFP4 items hold four weight
// blocks: the A loads, the same for every block of an item, then serve four
// times 16 rows of codes (two blocks: 0.84 -> 0.75 ms for GEMM1 at decode).
// Partial sums of the waves meet in LDS and wave 0 applies the epilogue.

template <int MB, int NB>
struct StreamFrag {
    uint4 b[NB][4];
    uint4 a[MB][4];
};

// The lane offset of an A row past the tile's valid rows: beyond the range
// of a raw buffer descriptor of 2^31 - 1 bytes, so the buffer load returns
// zeros (into registers or LDS) without touching memory.  Those rows'
// results are never stored; zero operands make their MFMAs cheap in power,
// and the chip's clock follows the power the MFMAs draw on these GEMMs.
constexpr uint32_t kPadRowOffset = 0x80000000u;

// Register-path loads are split in two: stream_fetch issues a K group's loads
// into raw registers (codes and scale bytes as stored), stream_decode turns
// them into MFMA fragments.  The loop decodes a group only when it needs it,
// with the next group's loads in flight: decoding right after issuing would
// make every group wait for its own loads.
template <int MB, int NB, bool MX, int AT>
struct StreamRaw {
    uint4 b[NB][MX ? 1 : 4];  // MXFP4: 32 E2M1 codes of the lane's block; else 4 x 8 values
    uint32_t bs[MX ? NB : 1];  // MXFP4: the block's E8M0 scale byte
    uint4 a[MB][AT == ACT_Q8 ? 2 : 4];  // MXFP8: 32 E4M3 codes; else 4 x 8 values
    uint32_t as[AT == ACT_Q8 ? MB : 1];  // MXFP8: the block's E8M0 scale byte
};

template <int MB, int NB, bool MX, int AT, bool ABUF>
__device__ __forceinline__ void stream_fetch(StreamRaw<MB, NB, MX, AT> &r, const uint8_t *const bptr[NB],
                                             const uint16_t *const aptr[MB],
                                             __amdgpu_buffer_rsrc_t ra, const uint32_t (&aoff)[MB],
                                             const uint8_t *const a8ptr[MB], const uint8_t *const a8scale[MB],
                                             int64_t kk) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        if constexpr (MX) {
            r.b[c][0] = *(const uint4 *)(bptr[c] + (kk >> 1));  // r.bs[c]: set by the caller (mx_scale)
        } else {
            const uint4 *p = (const uint4 *)(bptr[c] + kk * 2);
#pragma unroll
            for (int s = 0; s < 4; ++s) r.b[c][s] = p[s];
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        if constexpr (AT == ACT_Q8) {
            const uint4 *p = (const uint4 *)(a8ptr[m] + kk);
            r.a[m][0] = p[0];
            r.a[m][1] = p[1];
            r.as[m] = a8scale[m][kk >> 5];
        } else if constexpr (ABUF) {
            // rows past the tile's valid rows have an offset out of range: zeros, no memory access
#pragma unroll
            for (int s = 0; s < 4; ++s)
                r.a[m][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          ra, aoff[m], (uint32_t)(kk * 2 + s * 16), 0));
        } else {
            const uint4 *p = (const uint4 *)(aptr[m] + kk);
#pragma unroll
            for (int s = 0; s < 4; ++s) r.a[m][s] = p[s];
        }
    }
}

// MXFP4 scales on the register path.  A row keeps its E8M0 scales as K/32
// consecutive bytes, so the 32-bit word at byte 4G holds the scales of the
// four 32-element blocks of 128-wide group G, one per lane group.  Loaded
// byte by byte per group, every scale load touches as many cache lines as the
// group's code load (one per row) for a sixteenth of the bytes.  Instead a
// lane (q, li) loads, for up to 16 groups j of the wave's K range, the word
// of row li and group j into slot j / 4 when j % 4 == q, and a group's scale
// is read from lane (j % 4, li) with a cross-lane permute, byte lg.
constexpr int kMxWordGroups = 16;  // groups whose scale words the slots hold

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// (A vector indexed by the wave-uniform j / 4 stays in registers; selects
// between loads of an array would be folded into a load through a selected
// address, which keeps the array in scratch memory.)
__device__ __forceinline__ uint32_t mx_scale(u32x4_t w, int j, int li, int lg) {
    const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((((j & 3) << 4) + li) << 2, (int)w[(j >> 2) & 3]);
    return (v >> (8 * lg)) & 0xffu;
}

template <int MB, int NB, bool MX, int AT>
__device__ __forceinline__ void stream_decode(StreamFrag<MB, NB> &f, const StreamRaw<MB, NB, MX, AT> &r) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        if constexpr (MX) {
            f.b[c][0] = mxfp4x8_to_act<AT>(r.b[c][0].x, r.bs[c]);
            f.b[c][1] = mxfp4x8_to_act<AT>(r.b[c][0].y, r.bs[c]);
            f.b[c][2] = mxfp4x8_to_act<AT>(r.b[c][0].z, r.bs[c]);
            f.b[c][3] = mxfp4x8_to_act<AT>(r.b[c][0].w, r.bs[c]);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) f.b[c][s] = weight_bf16_as<AT>(r.b[c][s]);
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        if constexpr (AT == ACT_Q8) {
            mxfp8x16_to_bf16(r.a[m][0], r.as[m], f.a[m][0], f.a[m][1]);
            mxfp8x16_to_bf16(r.a[m][1], r.as[m], f.a[m][2], f.a[m][3]);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) f.a[m][s] = r.a[m][s];
        }
    }
}

// Items on bf16/fp16 weights (grouped 16-row tiles, dense 64-row tiles)
// stream their operands through LDS: a buffer load of 64 lanes x 16 bytes
// straight into LDS fills 8 rows x 128 bytes of one 64-wide K group (whole
// cache lines; weights with the non-temporal policy: a probe of this form
// streams at 7.0 TB/s against 6.2 for register loads in the lane pattern
// above, and reads L2-resident rows at 80-130 GB/s per CU against 36 for
// register loads).  Each wave keeps its K groups in three slots (each its
// own LDS object), a slot holding the group's MB 16-row A blocks and its NB
// 16-row B blocks.  Grouped slots (4 waves x 3 blocks x 2 KB) leave room
// for two workgroups per CU, so one covers the other's start and end of an
// item.  In a block, row r keeps logical chunk q (8 values) at chunk
// q ^ f(r), f(r) = (r >> 1) ^ 4 (r & 1): a fragment read (rows 0..15 at one
// logical chunk) then hits distinct 16-byte bank groups in every 8-lane and
// 16-lane phase.
constexpr int kStrmKG = 64;                            // K per group
constexpr int kStrmRow = kStrmKG * 2;                  // bytes per block row (128)
constexpr int kStrmBlock = 16 * kStrmRow;              // bytes per 16-row block (2 KB)
constexpr int kStrmLoads = kStrmBlock / 1024;          // loads per block (2)

template <int MB, int NB>
constexpr int strm_wave_bytes() { return (MB + NB) * kStrmBlock; }

__device__ __forceinline__ int strm_swz(int r) { return (r >> 1) ^ ((r & 1) << 2); }

// Slot S of a kernel whose waves hold MB A and NB B blocks per group.
template <int MB, int NB, int S>
__device__ __forceinline__ uint8_t *strm_slot() {
    __shared__ __attribute__((aligned(16))) uint8_t slot[4 * strm_wave_bytes<MB, NB>()];
    return slot;
}

// Per-item state of an LDS-streamed item: buffer descriptors of A (rows
// gathered: per-row lane offsets from the buffer start) and of the first
// row of each B block (rows consecutive); the lane's byte offsets of A load
// i (rows 8i + lane / 8) in aoff[i] and of B load i of a block in boff[i];
// the byte offsets (within a slot) of its fragment reads in roff[s].
constexpr int kStrmMaxMB = 4;  // A blocks per wave: 1 (grouped) or 4 (dense)
struct StrmCtx {
    __amdgpu_buffer_rsrc_t ra, rb0, rb1;
    uint32_t aoff[2 * kStrmMaxMB], boff[kStrmLoads], roff[kStrmKG / 32];
};

// A pointer the whole wave holds, moved to scalar registers (descriptors
// built from it then stay scalar).  Both halves are taken as unsigned: the
// builtin returns int, and a widened int would carry bit 31 of the low half
// into the high half.
__device__ __forceinline__ void *uniform_ptr(const void *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (void *)(((uint64_t)hi << 32) | lo);
}

// Loads of the K group at element kk into slot S (this wave's area): NA
// loads of 8 A rows each (fewer than 2 MB: the tile's rows fit in them),
// then the NB weight blocks.
template <int MB, int NB, int NA, int S>
__device__ __forceinline__ void strm_issue(const StrmCtx &c, int wave, int64_t kk) {
    // each access is one address step from its slot object, which keeps the
    // compiler's per-object tracking of these loads (and with it the freedom
    // to read other slots while they are in flight)
    uint8_t *const slot = strm_slot<MB, NB, S>();
    const int w0 = wave * strm_wave_bytes<MB, NB>();
#pragma unroll
    for (int i = 0; i < NA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.ra, MOE_LDS(slot + (w0 + i * 1024)), 16, c.aoff[i],
                                                 (int)(kk * 2), 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < kStrmLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(b == 0 ? c.rb0 : c.rb1,
                                                     MOE_LDS(slot + (w0 + (MB + b) * kStrmBlock + i * 1024)), 16,
                                                     c.boff[i], (int)(kk * 2), 0, kStreamPolicy);
}

// The order of a wave's K groups within an item's K slice (four waves, kq
// elements each): KO 1 = the wave's contiguous quarter, KO 4 = every fourth
// group from group `wave`.  kbeg is the wave's first group (strm_kbeg).
template <int KO>
__device__ __forceinline__ int64_t strm_kbeg(int64_t slice0, int64_t kq, int wave) {
    return KO == 4 ? slice0 + (int64_t)wave * kStrmKG : slice0 + wave * kq;
}
template <int KO>
__device__ __forceinline__ int64_t strm_kpos(int64_t kbeg, int g) {
    return kbeg + (int64_t)KO * kStrmKG * g;
}

// One K group g of an LDS-streamed item, slot S = g % 3.  On entry group g
// and (when g + 1 < ng) group g+1 are in flight, issued in that order.  The
// step waits for group g: all but the loads of group g+1 (NEXT), or for
// everything (last group); with ISSUE it then loads group g+2 into slot
// (S+2) % 3; it reads group g and runs its MFMAs.  Slot (S+2) % 3 last held
// group g-1, whose reads finished in the previous step.
template <int MB, int NB, int NA, int AT, int KO, int S, bool ISSUE, bool NEXT>
__device__ __forceinline__ void strm_step(floatx4_t (&acc)[MB][NB], const StrmCtx &c, int64_t kbeg, int g,
                                          int wave) {
    constexpr int NS = kStrmKG / 32;  // MFMA K steps per group
    // Loads of group g+1 left in flight: grouped items count one A load for
    // either A-block count, since the previous item may have issued this
    // item's first groups under the other count as far as the compiler can
    // tell (waiting for one more load of group g+1 costs nothing measurable).
    constexpr int kLeft = (MB == 1 ? 1 : NA) + NB * kStrmLoads;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NEXT ? kLeft : 0));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (ISSUE) strm_issue<MB, NB, NA, (S + 2) % 3>(c, wave, strm_kpos<KO>(kbeg, g + 2));
    const uint8_t *const slot = strm_slot<MB, NB, S>();
    uint4 fa[MB][NS], fb[NB][NS];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int s = 0; s < NS; ++s) fa[m][s] = *(const uint4 *)(slot + c.roff[s] + m * kStrmBlock);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < NS; ++s)
            fb[b][s] = weight_bf16_as<AT>(*(const uint4 *)(slot + c.roff[s] + (MB + b) * kStrmBlock));
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[m][b] = mfma16x16x32<AT>(fa[m][s], fb[b][s], acc[m][b]);
}

// The K loop of an LDS-streamed item over ng >= 2 groups from kbeg (K a
// multiple of 512): every group is loaded exactly once.  strm_first issues
// groups 0 and 1; strm_steps then runs the steady state in triples (each
// step issues the group two ahead) and the last 2..4 groups with the issues
// and waits that remain.
template <int MB, int NB, int NA, int KO>
__device__ __forceinline__ void strm_first(const StrmCtx &c, int wave, int64_t kbeg) {
    strm_issue<MB, NB, NA, 0>(c, wave, kbeg);
    strm_issue<MB, NB, NA, 1>(c, wave, strm_kpos<KO>(kbeg, 1));
}

template <int MB, int NB, int NA, int AT, int KO>
__device__ __forceinline__ void strm_steps(floatx4_t (&acc)[MB][NB], const StrmCtx &c, int64_t kbeg, int ng,
                                           int wave) {
    int g = 0;
    for (; g + 5 <= ng; g += 3) {
        strm_step<MB, NB, NA, AT, KO, 0, true, true>(acc, c, kbeg, g, wave);
        strm_step<MB, NB, NA, AT, KO, 1, true, true>(acc, c, kbeg, g + 1, wave);
        strm_step<MB, NB, NA, AT, KO, 2, true, true>(acc, c, kbeg, g + 2, wave);
    }
    switch (ng - g) {
    case 4:
        strm_step<MB, NB, NA, AT, KO, 0, true, true>(acc, c, kbeg, g, wave);
        strm_step<MB, NB, NA, AT, KO, 1, true, true>(acc, c, kbeg, g + 1, wave);
        strm_step<MB, NB, NA, AT, KO, 2, false, true>(acc, c, kbeg, g + 2, wave);
        strm_step<MB, NB, NA, AT, KO, 0, false, false>(acc, c, kbeg, g + 3, wave);
        break;
    case 3:
        strm_step<MB, NB, NA, AT, KO, 0, true, true>(acc, c, kbeg, g, wave);
        strm_step<MB, NB, NA, AT, KO, 1, false, true>(acc, c, kbeg, g + 1, wave);
        strm_step<MB, NB, NA, AT, KO, 2, false, false>(acc, c, kbeg, g + 2, wave);
        break;
    default:  // 2
        strm_step<MB, NB, NA, AT, KO, 0, false, true>(acc, c, kbeg, g, wave);
        strm_step<MB, NB, NA, AT, KO, 1, false, false>(acc, c, kbeg, g + 1, wave);
        break;
    }
}

template <int MB, int NB, int EPI, bool MX, bool GROUPED, int AT, int OT>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs a) {
    constexpr int BM = 16 * MB;
    __shared__ floatx4_t red[3][MB][NB][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15;  // row (A) / column (B) within a 16-block
    const int lg = lane >> 4;  // k group of 32 within a 128-wide K group

    const int64_t K = a.K;
    // dense fp32 outputs may split K into ks slices: slice s of an item adds
    // its partial sums into plane s of C ([ks][M][ldc])
    const int ks = (EPI == EPI_F32 && !MX && !GROUPED && a.ksplit > 1) ? a.ksplit : 1;
    const int64_t kq = K / ks / 4;       // K range of one wave
    // EPI_SWIGLU items hold kSwHalf gate blocks, then the matching up blocks
    constexpr int kSwHalf = NB > 1 ? NB / 2 : 1;
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / (16 * kSwHalf) : a.N / (16 * NB);
    const int ntiles = GROUPED ? *a.ntiles : (int)((a.M + BM - 1) / BM);
    const int64_t items = (int64_t)ntiles * nblocks * ks;

    // items on bf16/fp16 weights stream A and B through LDS
    constexpr bool kDma = !MX && NB <= 2 && (GROUPED ? MB == 1 : MB == 4);
    // The order of each wave's K groups, chosen by measurement at decode: the
    // four waves of a workgroup take every fourth group (so at any time they
    // read adjacent groups of the same rows) on the LDS path for GEMM1 (6%
    // faster than contiguous quarters) and the dense 16-bit projections (4%),
    // and on the register path for both grouped GEMMs (3% and 2%); GEMM2 on
    // the LDS path runs 12% slower that way and keeps contiguous quarters.
    constexpr int KO = (EPI == EPI_SWIGLU || (!GROUPED && EPI != EPI_F32)) ? 4 : 1;  // LDS path: 4 or 1
    constexpr int64_t kRegGS = GROUPED ? 512 : 128;  // register path: K stride of a wave's 128-wide groups
    // Cross-wave reduction and epilogue of one item (acc: this wave's partial sums).
    // EPI_NORM: the gains 1 + gamma of a lane's column in each block, loaded when the item is set up (a load
    // in the epilogue would hold the other waves at its barrier for a memory round trip per item)
    auto gains_of = [&](int64_t nb, float (&gam)[NB]) {
#pragma unroll
        for (int c = 0; c < NB; ++c)
            gam[c] = (EPI == EPI_NORM && a.gamma) ? 1.0f + a.gamma[(nb * NB + c) * 16 + li] : 1.0f;
    };
    auto finish = [&](const RowTile &rt, int64_t nb, int ksl, floatx4_t (&acc)[MB][NB], const float (&gam)[NB]) {
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
                float rowsq[NB][4];  // EPI_NORM: sums of squares per 16-column block and row
#pragma unroll
                for (int c = 0; c < NB; ++c)
#pragma unroll
                    for (int q = 0; q < 4; ++q) rowsq[c][q] = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int row = m * 16 + lg * 4 + q;
                    bool ok = row < rt.mcount;
                    int64_t p = rt.p0 + row;
                    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                        for (int c = 0; c < kSwHalf; ++c)
                            if (ok) {
                                float g = acc[m][c][q], u = acc[m][c + kSwHalf][q];
                                ((uint16_t *)a.C)[p * a.ldc + (nb * kSwHalf + c) * 16 + li] =
                                    f32_to_act<OT>(silu_fast(g) * u);
                            }
                    } else {
#pragma unroll
                        for (int c = 0; c < NB; ++c) {
                            int64_t n = (nb * NB + c) * 16 + li;
                            if constexpr (EPI == EPI_NORM) {
                                if (ok) {
                                    const uint16_t sv = f32_to_bf16(gam[c] * acc[m][c][q]);
                                    ((uint16_t *)a.C)[p * a.ldc + n] = sv;
                                    const float qv = a.norm_round ? bf16_to_f32(sv) : acc[m][c][q];
                                    rowsq[c][q] += qv * qv;
                                }
                            } else {
                                if (ok) rowsq[c][q] += store_elem<EPI, OT>(a, p + ksl * a.M, n, acc[m][c][q]);
                            }
                        }
                    }
                }
                if constexpr (EPI == EPI_NORM) {
#pragma unroll
                    for (int c = 0; c < NB; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            float v = sum16(rowsq[c][q]);
                            int row = m * 16 + lg * 4 + q;
                            if (li == 0 && row < rt.mcount) a.ssq[(rt.p0 + row) * a.nparts + nb * NB + c] = v;
                        }
                }
            }
        }
        __syncthreads();  // red[] is reused by the next item
    };

    if constexpr (kDma) {
        // LDS-streamed items run software-pipelined over the workgroup's items:
        // the first two K groups of the next item go out before this item's
        // reduction and epilogue, so they are in flight while those run.
        static_assert(MB <= kStrmMaxMB, "A blocks per wave");
        int64_t item = blockIdx.x;
        if (item >= items) return;
        // Lane-only offsets.  Load i fills rows r = 8i + lane / 8 (of the A blocks;
        // of a B block for i < 2); physical chunk lane % 8 holds logical chunk
        // (lane % 8) ^ f(r % 16).  Fragment reads take row li of the wave's blocks
        // at logical chunk 2 lg + s; each read offset is an opaque value, so every
        // read is one short address step from its slot object (the compiler then
        // knows which slot a read touches).
        StrmCtx c;
#pragma unroll
        for (int i = 0; i < kStrmLoads; ++i) {
            const int r = 8 * i + (lane >> 3);
            c.boff[i] = (uint32_t)(r * K * 2 + (((lane & 7) ^ strm_swz(r & 15)) << 4));
        }
#pragma unroll
        for (int s = 0; s < kStrmKG / 32; ++s) {
            c.roff[s] = (uint32_t)(wave * strm_wave_bytes<MB, NB>() + li * kStrmRow +
                                   ((((kStrmKG / 32) * lg + s) ^ strm_swz(li)) << 4));
            asm("" : "+v"(c.roff[s]));
        }
        struct Item {
            RowTile rt;
            int64_t nb, kbeg;
            int ksl;
            float gam[NB];
        };
        // the tile of item it and, for grouped items, its list entry
        auto tile_of = [&](int64_t it) { return (int)(it / ks / nblocks); };
        auto entry_of = [&](int64_t it) {
            TileEntry te{};
            if constexpr (GROUPED) te = a.tiles[tile_of(it)];
            return te;
        };
        // row tile, descriptors and A offsets of item it (te: its list entry)
        auto setup = [&](int64_t it, Item &I, const TileEntry &te) {
            I.ksl = (int)(it % ks);
            const int64_t tb = it / ks;
            const int t = (int)(tb / nblocks);
            I.nb = tb - (int64_t)t * nblocks;
            I.kbeg = strm_kbeg<KO>(I.ksl * 4 * kq, kq, wave);
            gains_of(I.nb, I.gam);
            if constexpr (GROUPED) {
                I.rt.e = te.e;
                I.rt.p0 = te.p0;
                I.rt.mcount = te.mcount;  // > 0 for every listed tile
            } else {
                load_tile(a, false, BM, t, I.rt);
            }
            // gathered A rows are addressed from the buffer start (the layer keeps that
            // buffer below 2 GiB), contiguous ones from the tile's first row
            const uint16_t *abase = a.a_gather ? a.A : a.A + I.rt.p0 * a.lda;
            c.ra = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(abase), 0, 0x7fffffff, 0x00020000);
#pragma unroll
            for (int i = 0; i < 2 * MB; ++i) {
                const int r = 8 * i + (lane >> 3);
                const int rr = min(r, I.rt.mcount - 1);  // rows past the valid ones read the last
                const int64_t arow = a.a_gather ? (int64_t)a.a_gather[I.rt.p0 + rr] : rr;
                c.aoff[i] = (uint32_t)(arow * a.lda * 2 + (((lane & 7) ^ strm_swz(r & 15)) << 4));
            }
            const int64_t brow0 = GROUPED ? (int64_t)I.rt.e * a.b_group_rows : 0;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                int64_t r0;
                if constexpr (EPI == EPI_SWIGLU)
                    r0 = brow0 + (b == 0 ? 0 : a.N) + I.nb * 16;
                else
                    r0 = brow0 + (I.nb * NB + b) * 16;
                const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const uint8_t *)a.B + r0 * K * 2),
                                                                    0, 0x7fffffff, 0x00020000);
                if (b == 0) c.rb0 = rsrc;
                else c.rb1 = rsrc;
            }
        };
        // Tiles of up to 8 rows (most of them at decode) load one A row block per
        // group: fragment rows 8..15 then hold stale data, and their results are
        // never stored.
        auto first = [&](const Item &I) {
            if constexpr (MB == 1) {
                if (I.rt.mcount <= 8) strm_first<MB, NB, 1, KO>(c, wave, I.kbeg);
                else strm_first<MB, NB, 2, KO>(c, wave, I.kbeg);
            } else {
                strm_first<MB, NB, 2 * MB, KO>(c, wave, I.kbeg);
            }
        };
        const int ng = (int)(kq / kStrmKG);
        Item cur;
        setup(item, cur, entry_of(item));
        first(cur);
        for (;;) {
            // the next item's list entry goes out now, under this item's K loop
            const int64_t nx = item + gridDim.x;
            const TileEntry te_nx = nx < items ? entry_of(nx) : TileEntry{};
            floatx4_t acc[MB][NB];
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[m][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (MB == 1) {
                if (cur.rt.mcount <= 8) strm_steps<MB, NB, 1, AT, KO>(acc, c, cur.kbeg, ng, wave);
                else strm_steps<MB, NB, 2, AT, KO>(acc, c, cur.kbeg, ng, wave);
            } else {
                strm_steps<MB, NB, 2 * MB, AT, KO>(acc, c, cur.kbeg, ng, wave);
            }
            // every load of this item has landed and every slot read is done
            Item nxt;
            if (nx < items) {
                setup(nx, nxt, te_nx);
                first(nxt);
            }
            finish(cur.rt, cur.nb, cur.ksl, acc, cur.gam);
            if (nx >= items) break;
            item = nx;
            cur = nxt;
        }
        return;
    }
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int ksl = (int)(item % ks);
        const int64_t tb = item / ks;
        const int t = (int)(tb / nblocks);
        const int64_t nb = tb - (int64_t)t * nblocks;
        // the wave's 128-wide K groups: its contiguous quarter (gs = 128) or
        // every fourth group from group `wave` (gs = 512)
        constexpr int64_t gs = kRegGS;
        const int64_t kbeg = gs == 128 ? (ksl * 4 + wave) * kq : ksl * 4 * kq + wave * 128;
        const int64_t kend = kbeg + (kq / 128) * gs;
        RowTile rt;
        load_tile(a, GROUPED, BM, t, rt);  // mcount > 0 for every listed tile
        float gam[NB];
        gains_of(nb, gam);

        // B row pointers (lane's row li of each 16-row block) and A row pointers.
        const uint8_t *bptr[NB];
        const uint8_t *srow[NB];  // MXFP4: the row's scale bytes
        int64_t brow0 = GROUPED ? (int64_t)rt.e * a.b_group_rows : 0;
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            int64_t r;
            if constexpr (EPI == EPI_SWIGLU)
                r = brow0 + (c < kSwHalf ? 0 : a.N) + (nb * kSwHalf + c % kSwHalf) * 16 + li;
            else
                r = brow0 + (nb * NB + c) * 16 + li;
            if constexpr (MX) {
                // lane group lg reads its 32-element block of each 128-wide group
                bptr[c] = (const uint8_t *)a.B + r * (K / 2) + (lg * 32) / 2;
                srow[c] = (const uint8_t *)a.B + a.b_rows_total * (K / 2) + r * (K / 32);
            } else {
                bptr[c] = (const uint8_t *)a.B + (r * K + lg * 32) * 2;
                srow[c] = nullptr;
            }
        }
        // A rows.  Grouped items (mostly a few valid rows of 16 at decode) read
        // 16-bit rows through a buffer descriptor (gathered rows from the buffer
        // start, which the layer keeps below 2 GiB; contiguous rows from the
        // tile's first row), rows past the tile's valid rows at an out-of-range
        // offset, so those lanes touch no memory.  Dense items and MXFP8 rows
        // read through pointers, rows past the valid ones at the last valid row
        // (their results are never stored).  Every lane issues the same loads,
        // so the in-order wait counts stay exact.
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(a.a_gather ? a.A : a.A + rt.p0 * a.lda), 0, 0x7fffffff, 0x00020000);
        uint32_t aoff[MB];
        const uint16_t *aptr[MB];
        const uint8_t *a8ptr[MB], *a8scale[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const int lrow = m * 16 + li;
            const int row = min(lrow, rt.mcount - 1);
            int64_t p = rt.p0 + row;
            int64_t arow = a.a_gather ? (int64_t)a.a_gather[p] : p;
            aoff[m] = 0;
            aptr[m] = nullptr;
            a8ptr[m] = a8scale[m] = nullptr;
            if constexpr (AT == ACT_Q8) {
                a8ptr[m] = a.A8 + arow * K + lg * 32;
                a8scale[m] = a.A8s + arow * (K / 32) + lg;
            } else if constexpr (GROUPED) {
                const int64_t lr = a.a_gather ? arow : row;
                aoff[m] = lrow < rt.mcount ? (uint32_t)((lr * a.lda + lg * 32) * 2) : kPadRowOffset;
            } else {
                aptr[m] = a.A + arow * a.lda + lg * 32;
            }
        }

        floatx4_t acc[MB][NB];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int c = 0; c < NB; ++c) acc[m][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        // Two groups in flight: the raw registers of groups g+1 and g+2 while group g's MFMAs run.  The
        // two raw buffers alternate by position in an unrolled pair of groups, each refilled once its
        // group's MFMAs have read it, so no buffer is copied (a copy of registers a load is still writing,
        // or a load into registers an MFMA has yet to read, would wait for that load).  MXFP4 items run
        // the pipeline over chunks of up to kMxWordGroups groups, each after loading its scale words.
        StreamRaw<MB, NB, MX, AT> r0, r1;
        for (int64_t kc = kbeg; kc < kend; kc += (MX ? kMxWordGroups * gs : kend - kbeg)) {
            const int64_t kce = MX ? min(kend, kc + kMxWordGroups * gs) : kend;
            u32x4_t sw[MX ? NB : 1];
            if constexpr (MX) {
                const int nw = (int)((kce - kc) / gs + 3) >> 2;  // words per lane (wave-uniform)
#pragma unroll
                for (int c = 0; c < NB; ++c)
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int64_t j = min((int64_t)(4 * h + lg), (kce - kc) / gs - 1);
                        sw[c][h] = h < nw ? *(const uint32_t *)(srow[c] + (((kc + j * gs) >> 7) << 2)) : 0u;
                    }
            }
            // the scales of the group at kn into the raw buffer o (its code loads may still be in flight)
            auto scales = [&](StreamRaw<MB, NB, MX, AT> &o, int64_t kn) {
                if constexpr (MX) {
                    const int j = (int)((kn - kc) / gs);
#pragma unroll
                    for (int c = 0; c < NB; ++c) o.bs[c] = mx_scale(sw[c], j, li, lg);
                }
            };
            auto step = [&](StreamRaw<MB, NB, MX, AT> &r, StreamRaw<MB, NB, MX, AT> &o, int64_t kk) {
                StreamFrag<MB, NB> cur;
                stream_decode<MB, NB, MX, AT>(cur, r);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int c = 0; c < NB; ++c)
                            acc[m][c] = mfma16x16x32<AT>(cur.a[m][s], cur.b[c][s], acc[m][c]);
                if (kk + 2 * gs < kce)
                    stream_fetch<MB, NB, MX, AT, GROUPED>(r, bptr, aptr, ra, aoff, a8ptr, a8scale, kk + 2 * gs);
                scales(o, kk + gs);  // the next group's, read while this group's MFMAs run
                // a group's refill stays ahead of the next group's, so waiting for one buffer leaves the
                // other's loads in flight (the counter is in order)
                __builtin_amdgcn_sched_barrier(0);
            };
            stream_fetch<MB, NB, MX, AT, GROUPED>(r0, bptr, aptr, ra, aoff, a8ptr, a8scale, kc);
            if (kc + gs < kce)
                stream_fetch<MB, NB, MX, AT, GROUPED>(r1, bptr, aptr, ra, aoff, a8ptr, a8scale, kc + gs);
            scales(r0, kc);
            int64_t kk = kc;
            for (; kk + 4 * gs <= kce; kk += 2 * gs) {  // every refill in range: one path, exact waits
                step(r0, r1, kk);
                step(r1, r0, kk + gs);
            }
            // the last 1..3 groups, already loaded or in flight
            step(r0, r1, kk);
            if (kk + gs < kce) step(r1, r0, kk + gs);
            if (kk + 2 * gs < kce) step(r0, r1, kk + 2 * gs);
        }

        finish(rt, nb, ksl, acc, gam);
    }
}

// ---------------------------------------------------------------------------
// Large-tile kernel (many rows per expert; dense projections at large T)
// ---------------------------------------------------------------------------
//
// Output tiles of 32 x 32 x 16 MFMA blocks, one wave per SIMD (four waves;
// eight for the wide mode): with one wave per SIMD this MFMA shape issues
// close to its peak rate, the 16 x 16 x 32 shape would need two.  K advances
// in pairs of 64: a K pair of A (activation) or B (weight) rows sits in LDS
// as 128-byte rows.  Operands move global -> LDS with buffer loads straight
// into LDS: a wave instruction fills 8 rows x 128 bytes in lane order, so
// each lane fetches the global chunk that belongs at its XOR-swizzled LDS
// slot and every L2 request is a whole 128-byte row segment.  A double-
// buffers and B rotates through three slots (the weight ring below); MXFP4
// slots hold codes and scale words that are dequantised in registers as the
// fragments are read, and bf16 weights under fp16 activations are converted
// per fragment in registers.  A pair runs as two 32-K sub-steps with
// fragments double-buffered in registers: the MFMAs of one overlap the LDS
// reads of the next, the loads of later pairs are spread between the MFMAs,
// and the only barrier of a pair sits in front of it.
// The MFMA operands are swapped (B first), so a lane's accumulator registers
// hold runs of four adjacent output columns of one row: epilogue stores are 8
// or 16 bytes wide.  EPI_SWIGLU tiles hold 128 gate rows then the 128 matching
// up rows; a wave's gate column blocks pair with its up column blocks.
// Rows past the tile's valid rows load zeros (an offset beyond the buffer
// descriptor's range); their results are never stored.

constexpr int kBigBM = kTileBM, kBigBN = kTileBN, kBigBK = 64;  // K per pair
static_assert(kBigBM == 256 && kBigBN == 256, "the wave layout below assumes 256x256 tiles");
constexpr int kBigRow = kBigBK * 2;                             // bytes per LDS row (128)

// 128-byte rows (64 x 16-bit): 16-byte chunk c of row r lives at chunk
// c ^ swz(r).  A fragment read takes one logical chunk of 32 consecutive
// rows (lanes 0-31) and the next chunk of the same rows (lanes 32-63).  Any
// 8 consecutive rows from a multiple of 8 get 8 distinct XOR terms, and of
// 16 rows from a multiple of 16 the even ones get 8 distinct terms and so do
// the odd ones, so a phase of 8 lanes over 128 bytes of banks and a phase of
// 16 lanes over 256 bytes both touch every 16-byte bank group once.
__host__ __device__ constexpr int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ int bswz(int row, int chunk) {
    return row * kBigRow + ((chunk ^ swz(row)) << 4);
}

// Tile modes: TM 0 = full (256 A rows x 256 B rows; 2 x 2 waves of 128 x 128),
// TM 1 = half (128 x 256; the four waves share the 128 A rows, each takes 64 B
// rows), TM 2 = tall (320 x 128; 2 x 2 waves of 160 x 64), TM 3 = wide
// (320 x 256; eight waves, two per SIMD, in 2 x 4 blocks of 160 x 64).  A
// grouped expert with at most 320 rows gets a single tile of the smallest
// mode that holds it, so its weights stream once: wide for bf16 and fp16
// weights (half the A re-reads of tall: 128 column blocks of GEMM1 instead
// of 256), tall for MXFP4 (whose dequantisation area leaves no LDS for wide).
template <int TM> struct BigTile {
    static constexpr int WAVES = TM == 3 ? 8 : 4;                  // waves per workgroup
    static constexpr int BM = TM == 0 ? 256 : TM == 1 ? 128 : 320;  // A rows per tile
    static constexpr int BN = TM == 2 ? 128 : 256;                  // B rows per tile
    static constexpr int MB = TM >= 2 ? 5 : 4;                      // 32-row blocks per wave
    static constexpr int NBK = TM == 0 ? 4 : 2;                     // 32-column blocks per wave
    static constexpr int NA = BM / (8 * WAVES);                     // A loads (8 rows) per wave per pair
    static constexpr int NBL = BN / (8 * WAVES);                    // bf16 B loads per wave per pair
    static constexpr int NBC = BN / 128;                            // MXFP4 code loads per wave per pair
    static constexpr int BPW = BN / WAVES;                          // B rows loaded by one wave
};

// Load addresses: a wave-uniform base plus a 32-bit byte offset per lane, so
// the loads take the scalar-base form and the per-lane state stays small.
struct BigCtx {
    const uint8_t *A;       // activation base (uniform)
    uint32_t aoff[12];      // byte offsets of this lane's A chunks at k = 0
    const uint8_t *B;       // first B row of the tile (bf16) or its code row (MXFP4) (uniform)
    uint32_t boff[8];       // bf16: this lane's B chunks; MXFP4: [0..1] codes, [2] scale word
    const uint8_t *bsc;     // MXFP4: scale base of the tile (uniform)
    __amdgpu_buffer_rsrc_t ra, rb;  // ring: buffer descriptors of A and of the tile's B rows (bf16, or MXFP4 codes)
    __amdgpu_buffer_rsrc_t rs;      // ring, MXFP4: descriptor of the tile's scale rows
};

// A raw buffer descriptor over ptr (stride 0, 2^31 - 1 bytes): buffer loads
// take the per-lane 32-bit offset in a VGPR and the pair offset in an SGPR,
// so the compiler cannot fold them into per-lane 64-bit addresses.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(const void *ptr) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(ptr), 0, 0x7fffffff, 0x00020000);
}


// bf16 weights under fp16 activations are converted per fragment in
// registers, between the MFMAs.
template <bool MX, int AT> constexpr bool kBigRegConvert = !MX && AT == ACT_F16;

// The MFMAs of one sub-step, K half by K half, so two MFMAs on one
// accumulator are MB * NBK instructions apart.
template <int AT, int TM>
__device__ __forceinline__ void big_mma(floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                        const uint4 (&fa)[2 * BigTile<TM>::MB], const uint4 (&fb)[2 * BigTile<TM>::NBK]) {
    using S = BigTile<TM>;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < S::MB; ++m)
#pragma unroll
            for (int c = 0; c < S::NBK; ++c) acc[m][c] = mfma32x32x16<AT>(fb[2 * c + h], fa[2 * m + h], acc[m][c]);
}


// ---------------------------------------------------------------------------
// bf16 weights: a three-slot weight ring.  Every weight byte comes from HBM
// once, and a CU's loads return in issue order, so the pair time is set by
// how far ahead of their use the weight loads go out.  The ring keeps A
// (activations, L2-resident) double-buffered and B (weights) in three slots:
// after the barrier of pair pr a wave issues A(pr+2) and then B(pr+3), so
// the wait of pair pr+1 (for A(pr+2), B(pr+2)) leaves only B(pr+3) in
// flight and the weights get two pair times to arrive instead of one.
// Each slot is an LDS object of its own, which keeps the compiler's
// DMA-versus-read dependence tracking exact.
constexpr int kRingB = 3;  // weight slots

#define MOE_RING_SLOTS(TM, ASZ, BSZ)                                              \
    __shared__ __attribute__((aligned(16))) uint8_t ring##TM##_a0[ASZ];          \
    __shared__ __attribute__((aligned(16))) uint8_t ring##TM##_a1[ASZ];          \
    __shared__ __attribute__((aligned(16))) uint8_t ring##TM##_b0[BSZ];          \
    __shared__ __attribute__((aligned(16))) uint8_t ring##TM##_b1[BSZ];          \
    __shared__ __attribute__((aligned(16))) uint8_t ring##TM##_b2[BSZ];
MOE_RING_SLOTS(0, 256 * kBigRow, 256 * kBigRow)  // full: 160 KiB
MOE_RING_SLOTS(1, 128 * kBigRow, 256 * kBigRow)  // half: 128 KiB
MOE_RING_SLOTS(2, 320 * kBigRow, 128 * kBigRow)  // tall: 128 KiB
MOE_RING_SLOTS(3, 320 * kBigRow, 256 * kBigRow)  // wide: two weight slots used, 144 KiB
#undef MOE_RING_SLOTS

// MXFP4 tiles: the weight slots hold the E2M1 codes (BN rows x 32 bytes per
// pair) and, after them, the scale words (4 waves x 64 words); the codes are
// dequantised in registers as the fragments are read.
#define MOE_MX_SLOTS(TM, ASZ, QSZ)                                                \
    __shared__ __attribute__((aligned(16))) uint8_t mx##TM##_a0[ASZ];            \
    __shared__ __attribute__((aligned(16))) uint8_t mx##TM##_a1[ASZ];            \
    __shared__ __attribute__((aligned(16))) uint8_t mx##TM##_q0[QSZ];            \
    __shared__ __attribute__((aligned(16))) uint8_t mx##TM##_q1[QSZ];            \
    __shared__ __attribute__((aligned(16))) uint8_t mx##TM##_q2[QSZ];
MOE_MX_SLOTS(0, 256 * kBigRow, 256 * 32 + 1024)  // full: 91 KiB
MOE_MX_SLOTS(1, 128 * kBigRow, 256 * 32 + 1024)  // half: 59 KiB
MOE_MX_SLOTS(2, 320 * kBigRow, 128 * 32 + 1024)  // tall: 95 KiB
#undef MOE_MX_SLOTS

template <int TM, int S, bool MX = false>
__device__ __forceinline__ uint8_t *ring_a() {
    static_assert(S == 0 || S == 1, "two activation slots");
    static_assert(!MX || TM <= 2, "MXFP4 tiles: full, half, tall");
    if constexpr (MX) {
        if constexpr (TM == 0) return S ? mx0_a1 : mx0_a0;
        else if constexpr (TM == 1) return S ? mx1_a1 : mx1_a0;
        else return S ? mx2_a1 : mx2_a0;
    } else if constexpr (TM == 0) return S ? ring0_a1 : ring0_a0;
    else if constexpr (TM == 1) return S ? ring1_a1 : ring1_a0;
    else if constexpr (TM == 2) return S ? ring2_a1 : ring2_a0;
    else return S ? ring3_a1 : ring3_a0;
}

template <int TM, int S, bool MX = false>
__device__ __forceinline__ uint8_t *ring_b() {
    static_assert(S >= 0 && S < (TM == 3 ? 2 : kRingB), "weight slot");
    static_assert(!MX || TM <= 2, "MXFP4 tiles: full, half, tall");
    if constexpr (MX) {
        if constexpr (TM == 0) return S == 0 ? mx0_q0 : S == 1 ? mx0_q1 : mx0_q2;
        else if constexpr (TM == 1) return S == 0 ? mx1_q0 : S == 1 ? mx1_q1 : mx1_q2;
        else return S == 0 ? mx2_q0 : S == 1 ? mx2_q1 : mx2_q2;
    } else if constexpr (TM == 0) return S == 0 ? ring0_b0 : S == 1 ? ring0_b1 : ring0_b2;
    else if constexpr (TM == 1) return S == 0 ? ring1_b0 : S == 1 ? ring1_b1 : ring1_b2;
    else if constexpr (TM == 2) return S == 0 ? ring2_b0 : S == 1 ? ring2_b1 : ring2_b2;
    else return S == 0 ? ring3_b0 : ring3_b1;
}

template <int TM, int S, bool MX = false>
__device__ __forceinline__ void ring_issue_a(const BigCtx &c, int pr, int wave) {
    using T = BigTile<TM>;
    uint8_t *buf = ring_a<TM, S, MX>();
#pragma unroll
    for (int i = 0; i < T::NA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.ra, MOE_LDS(buf + (wave * T::NA + i) * 1024), 16, c.aoff[i],
                                                 pr * kBigRow, 0, 0);
}

template <int TM, int S, bool MX = false>
__device__ __forceinline__ void ring_issue_b(const BigCtx &c, int pr, int wave) {
    using T = BigTile<TM>;
    uint8_t *buf = ring_b<TM, S, MX>();
    if constexpr (MX) {
        // codes: lane l of load i fills row BPW*wave + 32i + l/2, bytes 16(l&1) .. of pair pr
#pragma unroll
        for (int i = 0; i < T::NBC; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rb, MOE_LDS(buf + (wave * T::NBC + i) * 1024), 16, c.boff[i],
                                                     pr * 32, 0, kStreamPolicy);
        // the 4-byte-aligned word holding the scale bytes of K-tiles 2pr, 2pr+1
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, MOE_LDS(buf + T::BN * 32 + wave * 256), 4, c.boff[2],
                                                 (2 * pr) & ~3, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < T::NBL; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rb, MOE_LDS(buf + (wave * T::NBL + i) * 1024), 16, c.boff[i],
                                                     pr * kBigRow, 0, kStreamPolicy);
    }
}

// Fragments of sub-step HS of pair pr on an MXFP4 tile.  A lane's two 8-value
// halves h = 0, 1 of the sub-step cover K = 32HS + 16lh + 8h .. +7 (A and B
// alike, so the sums are unchanged): its 8 code bytes of a B row are
// contiguous, dequantised here with the row's scale of K-tile 2pr + HS.
template <int TM, int SA, int SB, int HS, int AT>
__device__ __forceinline__ void ring_read_mx(uint4 (&fa)[2 * BigTile<TM>::MB], uint4 (&fb)[2 * BigTile<TM>::NBK],
                                             const int (&bcol)[BigTile<TM>::NBK], int arow0, int lr, int lh,
                                             int pr) {
    using T = BigTile<TM>;
    const uint8_t *ab = ring_a<TM, SA, true>();
    const uint8_t *qb = ring_b<TM, SB, true>();
    const int sh = 8 * ((2 * pr + HS) & 3);
#pragma unroll
    for (int c = 0; c < T::NBK; ++c) {
        const int row = bcol[c] + lr;
        const uint2 cw = *(const uint2 *)(qb + row * 32 + HS * 16 + lh * 8);
        const uint32_t sw = *(const uint32_t *)(qb + T::BN * 32 + (row / T::BPW) * 256 + (row % T::BPW) * 4);
        const uint32_t e = (sw >> sh) & 255u;
        fb[2 * c] = mxfp4x8_to_act<AT>(cw.x, e);
        fb[2 * c + 1] = mxfp4x8_to_act<AT>(cw.y, e);
    }
#pragma unroll
    for (int m = 0; m < T::MB; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            fa[2 * m + h] = *(const uint4 *)(ab + bswz(arow0 + m * 32 + lr, 4 * HS + 2 * lh + h));
}

// Fragments of sub-step HS from activation slot SA and weight slot SB:
// lane (lr = l % 32, lh = l / 32) reads row lr of each 32-row block at
// logical chunks 4 * HS + 2h + lh (fa[2m + h]: A rows arow0 + 32m + lr;
// fb[2c + h]: B rows bcol[c] + lr).
template <int TM, int SA, int SB, int HS, bool CVT>
__device__ __forceinline__ void ring_read(uint4 (&fa)[2 * BigTile<TM>::MB], uint4 (&fb)[2 * BigTile<TM>::NBK],
                                          const int (&bcol)[BigTile<TM>::NBK], int arow0, int lr, int lh) {
    using T = BigTile<TM>;
    const uint8_t *ab = ring_a<TM, SA>();
    const uint8_t *bb = ring_b<TM, SB>();
#pragma unroll
    for (int c = 0; c < T::NBK; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 v = *(const uint4 *)(bb + bswz(bcol[c] + lr, 4 * HS + 2 * h + lh));
            fb[2 * c + h] = CVT ? bf16x8_to_f16x8(v) : v;
        }
#pragma unroll
    for (int m = 0; m < T::MB; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) fa[2 * m + h] = *(const uint4 *)(ab + bswz(arow0 + m * 32 + lr, 4 * HS + 2 * h + lh));
}

// Pair pr with A in slot SA = pr % 2 and B in slot SB = pr % 3.  On entry
// the wave holds the fragments of sub-step 2pr (f0), both slots are
// complete everywhere, and A(pr+1), B(pr+1), B(pr+2) are in flight, issued
// in the order B(pr+1), A(pr+1), B(pr+2).
//   first:  read sub-step 2pr+1 into f1; MFMAs on f0.
//   second: wait for the own A(pr+1) and B(pr+1) (all but the last NBL
//           loads), barrier (every read of slots SA and SB done), issue
//           A(pr+2) into SA and B(pr+3) into SB (clamped to the last pair:
//           clamped loads are never read), read sub-step 2pr+2 into f0,
//           MFMAs on f1 with the loads and reads spread between them.
template <int TM, int AT, int SA, int SB, bool MX = false>
__device__ __forceinline__ void ring_pair(const BigCtx &c, floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                          uint4 (&fa0)[2 * BigTile<TM>::MB], uint4 (&fb0)[2 * BigTile<TM>::NBK],
                                          uint4 (&fa1)[2 * BigTile<TM>::MB], uint4 (&fb1)[2 * BigTile<TM>::NBK],
                                          const int (&bcol)[BigTile<TM>::NBK], int pr, int npair, int wave, int arow0,
                                          int lane) {
    using T = BigTile<TM>;
    constexpr bool CVT = kBigRegConvert<false, AT>;
    constexpr int NBX = MX ? T::NBC + 1 : T::NBL;  // weight-side loads per wave per pair
    const int lr = lane & 31, lh = lane >> 5;
    if constexpr (MX) ring_read_mx<TM, SA, SB, 1, AT>(fa1, fb1, bcol, arow0, lr, lh, pr);
    else ring_read<TM, SA, SB, 1, CVT>(fa1, fb1, bcol, arow0, lr, lh);
    big_mma<AT, TM>(acc, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NBX));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    ring_issue_a<TM, SA, MX>(c, min(pr + 2, npair - 1), wave);
    ring_issue_b<TM, SB, MX>(c, min(pr + 3, npair - 1), wave);
    if constexpr (MX) ring_read_mx<TM, SA ^ 1, (SB + 1) % kRingB, 0, AT>(fa0, fb0, bcol, arow0, lr, lh, pr + 1);
    else ring_read<TM, SA ^ 1, (SB + 1) % kRingB, 0, CVT>(fa0, fb0, bcol, arow0, lr, lh);
    big_mma<AT, TM>(acc, fa1, fb1);
    // LDS reads first, so they land while the later MFMAs run and the wait
    // that ends the sub-step does not stall; the loads need not land soon
    constexpr int NL = T::NA + NBX, NR = 2 * (T::MB + T::NBK), NM = 2 * T::MB * T::NBK;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // direct-to-LDS load
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NL - NR > 0 ? NM - NL - NR : 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
}

// Wide tiles: eight waves, two per SIMD, so a wave holds 160 accumulators and
// the fragments of one 16-deep K slice (sub-step HS, half H) at a time; the
// other wave on its SIMD covers the LDS latency.  A and B are double-buffered
// in slot S = pr % 2: the pair's four quarters read slot S, then the wave
// waits for its own loads of pair pr+1, passes the barrier (pair pr+1
// complete everywhere, every read of slot S done) and issues pair pr+2 into
// slot S (clamped to the last pair: clamped loads are never read).
template <int TM, int S, int HS, int H, bool CVT, int MV>
__device__ __forceinline__ void wide_read(uint4 (&fa)[BigTile<TM>::MB], uint4 (&fb)[BigTile<TM>::NBK],
                                          const int (&bcol)[BigTile<TM>::NBK], int arow0, int lr, int lh) {
    using T = BigTile<TM>;
    const uint8_t *ab = ring_a<TM, S>();
    const uint8_t *bb = ring_b<TM, S>();
#pragma unroll
    for (int c = 0; c < T::NBK; ++c) {
        const uint4 v = *(const uint4 *)(bb + bswz(bcol[c] + lr, 4 * HS + 2 * H + lh));
        fb[c] = CVT ? bf16x8_to_f16x8(v) : v;
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) fa[m] = *(const uint4 *)(ab + bswz(arow0 + m * 32 + lr, 4 * HS + 2 * H + lh));
}

// Quarters are software-pipelined across two fragment buffers: the reads
// of quarter q+1 overlap the MFMAs of quarter q.  On entry q0 holds quarter
// 0 of pair pr.  Before the last quarter the wave waits for its loads of
// pair pr+1 and passes the barrier (pair pr+1 complete everywhere, every
// read of slot S done); the loads of pair pr+2 into slot S and the reads of
// quarter 0 of pair pr+1 then go out between the last quarter's MFMAs.
template <int TM, int AT, int MV>
__device__ __forceinline__ void wide_mma(floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                         const uint4 (&fa)[BigTile<TM>::MB], const uint4 (&fb)[BigTile<TM>::NBK]) {
#pragma unroll
    for (int m = 0; m < MV; ++m)
#pragma unroll
        for (int c = 0; c < BigTile<TM>::NBK; ++c) acc[m][c] = mfma32x32x16<AT>(fb[c], fa[m], acc[m][c]);
}

template <int NL, int NR, int NM>
__device__ __forceinline__ void wide_interleave() {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // direct-to-LDS load
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NL - NR > 0 ? NM - NL - NR : 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
}

template <int TM, int AT, int S, int MV>
__device__ __forceinline__ void wide_pair(const BigCtx &c, floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                          uint4 (&qa0)[BigTile<TM>::MB], uint4 (&qb0)[BigTile<TM>::NBK],
                                          uint4 (&qa1)[BigTile<TM>::MB], uint4 (&qb1)[BigTile<TM>::NBK],
                                          const int (&bcol)[BigTile<TM>::NBK], int pr, int npair, int wave,
                                          int arow0, int lr, int lh) {
    using T = BigTile<TM>;
    constexpr bool CVT = kBigRegConvert<false, AT>;
    constexpr int NR = MV + T::NBK, NM = MV * T::NBK;
    wide_read<TM, S, 0, 1, CVT, MV>(qa1, qb1, bcol, arow0, lr, lh);
    wide_mma<TM, AT, MV>(acc, qa0, qb0);
    wide_interleave<0, NR, NM>();
    wide_read<TM, S, 1, 0, CVT, MV>(qa0, qb0, bcol, arow0, lr, lh);
    wide_mma<TM, AT, MV>(acc, qa1, qb1);
    wide_interleave<0, NR, NM>();
    wide_read<TM, S, 1, 1, CVT, MV>(qa1, qb1, bcol, arow0, lr, lh);
    wide_mma<TM, AT, MV>(acc, qa0, qb0);
    wide_interleave<0, NR, NM>();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    ring_issue_a<TM, S>(c, min(pr + 2, npair - 1), wave);
    ring_issue_b<TM, S>(c, min(pr + 2, npair - 1), wave);
    wide_read<TM, S ^ 1, 0, 0, CVT, MV>(qa0, qb0, bcol, arow0, lr, lh);
    wide_mma<TM, AT, MV>(acc, qa1, qb1);
    wide_interleave<T::NA + T::NBL, NR, NM>();
}

// MV: the wave's 32-row blocks that hold valid rows (the others are padding:
// their fragments are not read and their MFMAs not issued).
template <int TM, int AT, int MV>
__device__ __forceinline__ void wide_kloop(const BigCtx &c, floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                           const int (&bcol)[BigTile<TM>::NBK], int npair, int wave, int arow0,
                                           int lane) {
    using T = BigTile<TM>;
    const int lr = lane & 31, lh = lane >> 5;
    ring_issue_a<TM, 0>(c, 0, wave);
    ring_issue_b<TM, 0>(c, 0, wave);
    ring_issue_a<TM, 1>(c, 1, wave);
    ring_issue_b<TM, 1>(c, 1, wave);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(T::NA + T::NBL));  // A(0) and B(0) landed
    __builtin_amdgcn_s_barrier();
    uint4 qa0[T::MB], qb0[T::NBK], qa1[T::MB], qb1[T::NBK];
    wide_read<TM, 0, 0, 0, kBigRegConvert<false, AT>, MV>(qa0, qb0, bcol, arow0, lr, lh);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    for (int pr = 0; pr < npair; pr += 2) {
        wide_pair<TM, AT, 0, MV>(c, acc, qa0, qb0, qa1, qb1, bcol, pr, npair, wave, arow0, lr, lh);
        wide_pair<TM, AT, 1, MV>(c, acc, qa0, qb0, qa1, qb1, bcol, pr + 1, npair, wave, arow0, lr, lh);
    }
}

// The K loop of a bf16 tile on the ring: prologue, then pairs in groups of
// six (one full turn of both slot cycles) and a tail of 0, 2 or 4 pairs
// (npair is a multiple of 8).
template <int TM, int AT, bool MX = false>
__device__ __forceinline__ void ring_kloop(const BigCtx &c, floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                           const int (&bcol)[BigTile<TM>::NBK], int npair, int wave, int arow0,
                                           int lane) {
    using T = BigTile<TM>;
    constexpr int MB = T::MB, NBK = T::NBK;
    const int lr = lane & 31, lh = lane >> 5;
    constexpr int NBX = MX ? T::NBC + 1 : T::NBL;  // weight-side loads per wave per pair
    ring_issue_a<TM, 0, MX>(c, 0, wave);
    ring_issue_b<TM, 0, MX>(c, 0, wave);
    ring_issue_b<TM, 1, MX>(c, 1, wave);
    ring_issue_a<TM, 1, MX>(c, 1, wave);
    ring_issue_b<TM, 2, MX>(c, 2, wave);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NBX + T::NA));  // A(0) and B(0) landed
    __builtin_amdgcn_s_barrier();
    uint4 fa0[2 * MB], fb0[2 * NBK], fa1[2 * MB], fb1[2 * NBK];
    if constexpr (MX) ring_read_mx<TM, 0, 0, 0, AT>(fa0, fb0, bcol, arow0, lr, lh, 0);
    else ring_read<TM, 0, 0, 0, kBigRegConvert<false, AT>>(fa0, fb0, bcol, arow0, lr, lh);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    int pr = 0;
    for (; pr + 6 <= npair; pr += 6) {
        ring_pair<TM, AT, 0, 0, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 0, npair, wave, arow0, lane);
        ring_pair<TM, AT, 1, 1, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 1, npair, wave, arow0, lane);
        ring_pair<TM, AT, 0, 2, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 2, npair, wave, arow0, lane);
        ring_pair<TM, AT, 1, 0, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 3, npair, wave, arow0, lane);
        ring_pair<TM, AT, 0, 1, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 4, npair, wave, arow0, lane);
        ring_pair<TM, AT, 1, 2, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 5, npair, wave, arow0, lane);
    }
    // Nested, so the second tail block has one predecessor and the compiler
    // knows exactly which slots have loads in flight when it starts.
    if (pr + 2 <= npair) {
        ring_pair<TM, AT, 0, 0, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 0, npair, wave, arow0, lane);
        ring_pair<TM, AT, 1, 1, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 1, npair, wave, arow0, lane);
        if (pr + 4 <= npair) {
            ring_pair<TM, AT, 0, 2, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 2, npair, wave, arow0, lane);
            ring_pair<TM, AT, 1, 0, MX>(c, acc, fa0, fb0, fa1, fb1, bcol, pr + 3, npair, wave, arow0, lane);
        }
    }
}

// B rows of a tile and how many column blocks a row of C has, per mode.
template <int EPI, int TM>
__host__ __device__ constexpr int64_t big_nblocks(int64_t N) {
    return (EPI == EPI_SWIGLU) ? N / (BigTile<TM>::BN / 2) : N / BigTile<TM>::BN;
}

// An opaque copy of a value: the compiler must recompute whatever derives
// from it after this point.  Lane-derived addresses and row indices are
// cheap to recompute but were otherwise hoisted to the kernel entry, held
// across the K loop and spilled; reloading a spill waits for every earlier
// memory operation of the wave, the epilogue's stores included.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// A tile entry read from the device-side list is the same in every lane;
// saying so keeps the tile's weight base in scalar registers, so the weight
// loads take the scalar-base form.
__device__ __forceinline__ void uniform_tile(RowTile &rt) {
    rt.e = __builtin_amdgcn_readfirstlane(rt.e);
    rt.mcount = __builtin_amdgcn_readfirstlane(rt.mcount);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)rt.p0);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)rt.p0 >> 32));
    rt.p0 = (int64_t)(((uint64_t)hi << 32) | lo);
}

template <int EPI, int OT, int TM>
__device__ __forceinline__ void big_epilogue(const GemmArgs &a, const RowTile &rt, int64_t nb,
                                             floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                             const int (&bcol)[BigTile<TM>::NBK], int arow0, int lane,
                                             int64_t coff);

// One output tile (row tile rt, column block nb, K slice ksl) in mode TM.
template <int EPI, bool MX, bool GROUPED, int AT, int OT, int TM>
__device__ __forceinline__ void big_item(const GemmArgs &a, const RowTile &rt, int64_t nb, int ksl, int wave,
                                         int lane) {
    using S = BigTile<TM>;
    constexpr int MB = S::MB, NBK = S::NBK, NA = S::NA;
    constexpr int WCOLS = 32 * NBK;       // B rows per wave (SWIGLU: half gate, half up)
    static_assert(!(MX && TM == 3), "MXFP4 grouped tiles use the tall mode");
    const int wm = TM == 1 ? 0 : TM == 3 ? wave >> 2 : wave >> 1;
    const int wn = TM == 1 ? wave : TM == 3 ? wave & 3 : wave & 1;
    const int arow0 = wm * 32 * MB;       // first A row of this wave's row blocks
    lane = opaque(lane);
    const int64_t K = a.K;                // B row length
    const int ks = (EPI == EPI_F32 && !MX && !GROUPED && a.ksplit > 1) ? a.ksplit : 1;
    const int64_t kn = K / ks, k0 = (int64_t)ksl * kn;  // this item's K slice
    const int npair = (int)(kn / kBigBK);  // a multiple of 8
    // Direct-load lane mapping of 128-byte rows: load q of a wave fills LDS
    // rows 8q .. 8q + 7, lane l row 8q + (l >> 3) at physical chunk l & 7,
    // i.e. logical chunk (l & 7) ^ swz(8q + (l >> 3)).
    const int drow = lane >> 3;
    auto dchunk = [&](int ldsrow) { return (lane & 7) ^ swz(ldsrow); };
    const int64_t brow0 = GROUPED ? (int64_t)rt.e * a.b_group_rows : 0;

    // Tile B rows of this wave's column blocks.  SWIGLU: the tile's first BN/2
    // B rows are gate rows, the rest the matching up rows; blocks c < NBK/2
    // are gate blocks and pair with block c + NBK/2.
    int bcol[NBK];
#pragma unroll
    for (int c = 0; c < NBK; ++c) {
        if constexpr (EPI == EPI_SWIGLU)
            bcol[c] = (c < NBK / 2) ? wn * (WCOLS / 2) + c * 32 : S::BN / 2 + wn * (WCOLS / 2) + (c - NBK / 2) * 32;
        else
            bcol[c] = wn * WCOLS + c * 32;
    }

    BigCtx c;
    // The loads take 32-bit lane offsets from the A base: gathered rows count
    // from the buffer start (the layer keeps the gathered latent rows below
    // 2 GiB), contiguous rows from the tile's first row, so a batch whose rows
    // span more than 2 GiB (GEMM2's T k rows) still addresses every row.
    c.A = (const uint8_t *)uniform_ptr(a.a_gather ? a.A : a.A + rt.p0 * a.lda) + k0 * 2;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int lrow = wave * (NA * 8) + i * 8 + drow;  // LDS row; rows past the valid ones load zeros
        const int row = min(lrow, rt.mcount - 1);
        const int64_t arow = a.a_gather ? (int64_t)a.a_gather[rt.p0 + row] : row;
        c.aoff[i] = lrow < rt.mcount ? (uint32_t)((arow * a.lda + dchunk(lrow) * 8) * 2) : kPadRowOffset;
    }
#pragma unroll
    for (int i = NA; i < 12; ++i) c.aoff[i] = 0;
    // The tile's B rows 0..BN-1: SWIGLU rows 0..BN/2-1 are gate rows
    // nb*BN/2.., the rest the matching up rows N + nb*BN/2..; a wave loads
    // tile rows BPW*wave + 8i + drow (bf16), codes of rows BPW*wave + 32i +
    // lane/2 and the scale words of rows BPW*wave + lane % BPW (MXFP4).
    const int64_t bfirst = brow0 + ((EPI == EPI_SWIGLU) ? nb * (S::BN / 2) : nb * S::BN);
    const int64_t upskip = (EPI == EPI_SWIGLU) ? a.N - S::BN / 2 : 0;  // up rows sit this far further on
    auto brel = [&](int row) -> int64_t { return row + (row >= S::BN / 2 ? upskip : 0); };
    if constexpr (MX) {
        c.B = (const uint8_t *)a.B + bfirst * (K / 2);
        c.bsc = (const uint8_t *)a.B + a.b_rows_total * (K / 2) + bfirst * (K / 32);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            c.boff[i] = i < S::NBC ? (uint32_t)(brel(wave * S::BPW + i * 32 + (lane >> 1)) * (K / 2) + (lane & 1) * 16) : 0;
        c.boff[2] = (uint32_t)(brel(wave * S::BPW + lane % S::BPW) * (K / 32));
#pragma unroll
        for (int i = 3; i < 8; ++i) c.boff[i] = 0;
        c.ra = ring_rsrc(c.A);
        c.rb = ring_rsrc(c.B);
        c.rs = ring_rsrc(c.bsc);
    } else {
        c.B = (const uint8_t *)((const uint16_t *)a.B + bfirst * K + k0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c.boff[i] = i < S::NBL ? (uint32_t)((brel(wave * S::BPW + i * 8 + drow) * K +
                                                 dchunk(wave * S::BPW + i * 8 + drow) * 8) * 2)
                                   : 0;
        c.bsc = nullptr;
        c.ra = ring_rsrc(c.A);
        c.rb = ring_rsrc(c.B);
    }

    floatx16_t acc[MB][NBK];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int cc = 0; cc < NBK; ++cc)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][cc][r] = 0.f;

    if constexpr (TM == 3) {
        // A wide tile holds 257..320 rows, so the second row of waves has 97..160 of them: its last
        // 32-row block is often all padding, and skipping it frees a tenth of its SIMD's MFMA time
        // (each SIMD runs one wave of each row).
        if (rt.mcount - arow0 > 32 * (MB - 1)) wide_kloop<TM, AT, MB>(c, acc, bcol, npair, wave, arow0, lane);
        else wide_kloop<TM, AT, MB - 1>(c, acc, bcol, npair, wave, arow0, lane);
    } else {
        ring_kloop<TM, AT, MX>(c, acc, bcol, npair, wave, arow0, lane);
    }
    // Drain the clamped tail loads before the buffers are refilled.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    big_epilogue<EPI, OT, TM>(a, rt, nb, acc, bcol, arow0, opaque(lane), ksl * a.M * a.ldc);
}

// Epilogue of one tile (lane id recomputed after the K loop).
template <int EPI, int OT, int TM>
__device__ __forceinline__ void big_epilogue(const GemmArgs &a, const RowTile &rt, int64_t nb,
                                             floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                             const int (&bcol)[BigTile<TM>::NBK], int arow0, int lane,
                                             int64_t coff) {
    using S = BigTile<TM>;
    constexpr int MB = S::MB, NBK = S::NBK;
    const int lr = lane & 31, lh = lane >> 5;
    // Epilogue: lane (lr, lh) holds, in block (m, c), output row arow0 + 32m +
    // lr and the tile columns bcol[c] + 8g + 4lh + q in register 4g + q
    // (g, q = 0..3): four runs of four adjacent columns.
    //
    // A load issued after a store waits for that store (one in-order memory
    // counter), so the loads the epilogue needs go out in batches ahead of
    // the stores: the norm gain 1 + gamma before the first store, the
    // residual rows and gate of block m before the stores of block m (one
    // wait per row block).
    constexpr bool kCol = EPI == EPI_NORM;
    float4 colv[kCol ? NBK : 1][4];
    if constexpr (kCol) {
#pragma unroll
        for (int cc = 0; cc < NBK; ++cc)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t n = nb * S::BN + bcol[cc] + 8 * g + 4 * lh;
                float4 gm = make_float4(0.f, 0.f, 0.f, 0.f);
                if (a.gamma) gm = *(const float4 *)(a.gamma + n);
                colv[cc][g] = make_float4(1.0f + gm.x, 1.0f + gm.y, 1.0f + gm.z, 1.0f + gm.w);
            }
    }
    constexpr bool kRes = EPI == EPI_RESID;
    uint2 resid[kRes ? NBK : 1][4];
    float4 gate[kRes ? NBK : 1][4];
    // residual and gate of row block m (rows past the tile's valid rows read its last valid row)
    auto load_resid = [&](int m) {
        const int64_t p = rt.p0 + min(arow0 + m * 32 + lr, rt.mcount - 1);
#pragma unroll
        for (int cc = 0; cc < NBK; ++cc)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t n = nb * S::BN + bcol[cc] + 8 * g + 4 * lh;
                resid[cc][g] = *(const uint2 *)(a.resid + p * a.N + n);
                gate[cc][g] = *(const float4 *)(a.gate + n);
            }
    };
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int row = arow0 + m * 32 + lr;
        const bool ok = row < rt.mcount;
        const int64_t p = rt.p0 + row;
        if constexpr (kRes) {
            // keeps the compiler from hoisting every block's loads to the top
            // (the residual and the output have different types)
            asm volatile("" ::: "memory");
            load_resid(m);
        }
        // The residual, norm and 16-bit-store epilogues: the block's
        // accumulators stay in their AGPRs up to here, so the VGPR copies the
        // arithmetic needs are made one row block at a time (copied all at
        // once after the K loop, they spilled).  The wide mode keeps its
        // accumulators in VGPRs.
        if constexpr (EPI != EPI_SWIGLU && EPI != EPI_F32 && TM != 3) {
#pragma unroll
            for (int cc = 0; cc < NBK; ++cc) asm volatile("" : "+a"(acc[m][cc]));
        }
        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int cc = 0; cc < NBK / 2; ++cc) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if (ok) {
                        uint16_t h[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            h[q] = f32_to_act<OT>(silu_fast(acc[m][cc][4 * g + q]) * acc[m][cc + NBK / 2][4 * g + q]);
                        const int64_t j = nb * (S::BN / 2) + bcol[cc] + 8 * g + 4 * lh;
                        *(uint2 *)((uint16_t *)a.C + p * a.ldc + j) =
                            make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                    }
                }
            }
        } else {
#pragma unroll
            for (int cc = 0; cc < NBK; ++cc) {
                const int64_t n0 = nb * S::BN + bcol[cc];
                float sq[2] = {0.f, 0.f};  // EPI_NORM: sums of squares of the two 16-column halves
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t n = n0 + 8 * g + 4 * lh;
                    floatx4_t v;
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = acc[m][cc][4 * g + q];
                    if constexpr (EPI == EPI_F32) {
                        if (ok) *(floatx4_t *)((float *)a.C + coff + p * a.ldc + n) = v;
                    } else if constexpr (EPI == EPI_ACT) {
                        if (ok)
                            *(uint2 *)((uint16_t *)a.C + p * a.ldc + n) =
                                make_uint2(f32_to_act<OT>(v[0]) | ((uint32_t)f32_to_act<OT>(v[1]) << 16),
                                           f32_to_act<OT>(v[2]) | ((uint32_t)f32_to_act<OT>(v[3]) << 16));
                    } else if constexpr (EPI == EPI_NORM) {
                        const float4 gs = colv[cc][g];
                        const float gq[4] = {gs.x, gs.y, gs.z, gs.w};
                        uint16_t h[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            h[q] = f32_to_bf16(gq[q] * v[q]);
                            const float e = a.norm_round ? bf16_to_f32(h[q]) : v[q];
                            sq[g >> 1] += e * e;
                        }
                        if (ok)
                            *(uint2 *)((uint16_t *)a.C + p * a.ldc + n) =
                                make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                    } else {  // EPI_RESID
                        if (ok) {
                            const uint2 hx = resid[cc][g];
                            const float4 gt = gate[cc][g];
                            floatx4_t o;
                            o[0] = bf16_to_f32((uint16_t)hx.x) + gt.x * v[0];
                            o[1] = bf16_to_f32((uint16_t)(hx.x >> 16)) + gt.y * v[1];
                            o[2] = bf16_to_f32((uint16_t)hx.y) + gt.z * v[2];
                            o[3] = bf16_to_f32((uint16_t)(hx.y >> 16)) + gt.w * v[3];
                            *(floatx4_t *)((float *)a.C + p * a.ldc + n) = o;
                            if (a.y) *(floatx4_t *)(a.y + p * a.N + n) = v;
                        }
                    }
                }
                if constexpr (EPI == EPI_NORM) {
                    // lanes lr and lr + 32 hold the other columns of each 16-column half
                    sq[0] += __shfl_xor(sq[0], 32, 64);
                    sq[1] += __shfl_xor(sq[1], 32, 64);
                    if (ok && lh == 0) {
                        a.ssq[p * a.nparts + n0 / 16] = sq[0];
                        a.ssq[p * a.nparts + n0 / 16 + 1] = sq[1];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large tiles on MXFP8 activations x MXFP4 weights (ACT_Q8): the scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 with operand a = 32 weight rows of E2M1
// codes and operand b = 32 activation rows of E4M3 codes (the swap keeps the
// accumulator layout, and so the epilogues, of the bf16 tiles); each lane
// gives 32 consecutive K values of one row of each operand and the E8M0 scale
// of that 32-block.  The products are exact and accumulate in fp32, so the
// tile computes what the bf16 tiles compute on the dequantised values, up to
// the order of the fp32 sums.
//
// K advances in steps of 128: a step of an activation row is 128 E4M3 bytes
// (an LDS row like a bf16 K pair, same swizzle and DMA pattern), a step of a
// weight row 64 bytes of E2M1 codes, and each row's four E8M0 scale bytes of
// the step are one 32-bit word.  Activations double-buffer, weights cycle
// through three slots (the ring of the bf16 tiles); every slot holds its
// rows' scale words after the codes, padded to whole 64-row loads so every
// wave issues the same loads.  A step runs as two 64-K sub-steps, the reads
// of one overlapping the MFMAs of the other.
// ---------------------------------------------------------------------------

constexpr int kQ8BK = 128;      // K per step
constexpr int kQ8BRow = 64;     // bytes of a weight row per step (E2M1 codes)

// 64-byte weight rows: 16-byte chunk c of row r lives at chunk c ^ q8_bswz(r).
// A fragment read takes one chunk of 32 consecutive rows (lanes 0-31) and the
// next chunk of the same rows (lanes 32-63); of any 8 consecutive rows from a
// multiple of 8 the even and the odd ones get 4 distinct terms each, and of
// any 16 rows from a multiple of 16 the rows of one residue mod 4 do, so an
// 8-lane phase over 128 bytes of banks and a 16-lane phase over 256 bytes
// both touch every 16-byte bank group once.
__host__ __device__ constexpr int q8_bswz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

template <int TM> struct Q8Tile {
    using B = BigTile<TM>;
    static_assert(TM <= 2, "MXFP8 tiles: full, half, tall");
    static constexpr int NA = B::BM / 32;                 // activation code loads (8 rows) per wave per step
    static constexpr int NAS = (B::BM + 255) / 256;       // activation scale loads (64 rows) per wave per step
    static constexpr int NBL = B::BN / 64;                // weight code loads (16 rows) per wave per step
    static constexpr int NBX = NBL + 1;                   // weight-side loads per wave per step (codes + scales)
    static constexpr int ASZ = B::BM * kBigRow + NAS * 1024;   // activation slot: codes, then scale words
    static constexpr int BSZ = B::BN * kQ8BRow + 1024;          // weight slot: codes, then scale words
};

#define MOE_Q8_SLOTS(TM)                                                                          \
    __shared__ __attribute__((aligned(16))) uint8_t q8##TM##_a0[Q8Tile<TM>::ASZ];                \
    __shared__ __attribute__((aligned(16))) uint8_t q8##TM##_a1[Q8Tile<TM>::ASZ];                \
    __shared__ __attribute__((aligned(16))) uint8_t q8##TM##_b0[Q8Tile<TM>::BSZ];                \
    __shared__ __attribute__((aligned(16))) uint8_t q8##TM##_b1[Q8Tile<TM>::BSZ];                \
    __shared__ __attribute__((aligned(16))) uint8_t q8##TM##_b2[Q8Tile<TM>::BSZ];
MOE_Q8_SLOTS(0)  // full: 2 x 33 KiB + 3 x 17 KiB
MOE_Q8_SLOTS(1)  // half: 2 x 17 KiB + 3 x 17 KiB
MOE_Q8_SLOTS(2)  // tall: 2 x 42 KiB + 3 x 9 KiB
#undef MOE_Q8_SLOTS

template <int TM, int S>
__device__ __forceinline__ uint8_t *q8_a() {
    static_assert(S == 0 || S == 1, "two activation slots");
    if constexpr (TM == 0) return S ? q80_a1 : q80_a0;
    else if constexpr (TM == 1) return S ? q81_a1 : q81_a0;
    else return S ? q82_a1 : q82_a0;
}

template <int TM, int S>
__device__ __forceinline__ uint8_t *q8_b() {
    static_assert(S >= 0 && S < kRingB, "weight slot");
    if constexpr (TM == 0) return S == 0 ? q80_b0 : S == 1 ? q80_b1 : q80_b2;
    else if constexpr (TM == 1) return S == 0 ? q81_b0 : S == 1 ? q81_b1 : q81_b2;
    else return S == 0 ? q82_b0 : S == 1 ? q82_b1 : q82_b2;
}

// Load state of a tile: descriptors of the activation codes, activation
// scales, weight codes and weight scales, and the lane's 32-bit offsets
// (at step 0) of each of its loads.
struct Q8Ctx {
    __amdgpu_buffer_rsrc_t ra, ras, rb, rbs;
    uint32_t aoff[10], asoff[2], boff[4], bsoff;
};

template <int TM, int S>
__device__ __forceinline__ void q8_issue_a(const Q8Ctx &c, int st, int wave) {
    using Q = Q8Tile<TM>;
    uint8_t *buf = q8_a<TM, S>();
#pragma unroll
    for (int i = 0; i < Q::NA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.ra, MOE_LDS(buf + (wave * Q::NA + i) * 1024), 16, c.aoff[i],
                                                 st * kQ8BK, 0, 0);
#pragma unroll
    for (int i = 0; i < Q::NAS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.ras, MOE_LDS(buf + BigTile<TM>::BM * kBigRow + (wave + 4 * i) * 256),
                                                 4, c.asoff[i], st * 4, 0, 0);
}

template <int TM, int S>
__device__ __forceinline__ void q8_issue_b(const Q8Ctx &c, int st, int wave) {
    using Q = Q8Tile<TM>;
    uint8_t *buf = q8_b<TM, S>();
#pragma unroll
    for (int i = 0; i < Q::NBL; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rb, MOE_LDS(buf + (wave * Q::NBL + i) * 1024), 16, c.boff[i],
                                                 st * kQ8BRow, 0, kStreamPolicy);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rbs, MOE_LDS(buf + BigTile<TM>::BN * kQ8BRow + wave * 256), 4, c.bsoff,
                                             st * 4, 0, 0);
}

typedef int int32x8_t __attribute__((ext_vector_type(8)));

// Fragments of sub-step HS (K 64 HS .. 64 HS + 63 of the step).  The scaled
// MFMA takes an E2M1 operand as 32 consecutive K values per lane (lane half
// lh: the 32-block lh of the 64) and an E4M3 operand as two runs of 16 (lane
// half lh: K 16 lh .. +15 of block 0, then of block 1), and applies to row i
// of block b the scale held by lane i + 32 b (checked on the chip with a
// one-wave probe).  So a lane reads weight rows bcol[c] + lr at chunk 2 HS +
// lh of the 64-byte row and activation rows arow0 + 32m + lr at chunks
// 4 HS + lh and 4 HS + 2 + lh of the 128-byte row, and gives the scales of
// block lh of the sub-step.
template <int TM, int SA, int SB, int HS>
__device__ __forceinline__ void q8_read(int32x8_t (&fa)[BigTile<TM>::MB], int32x8_t (&fb)[BigTile<TM>::NBK],
                                        const int (&bcol)[BigTile<TM>::NBK], int arow0, int lr, int lh) {
    using T = BigTile<TM>;
    const uint8_t *ab = q8_a<TM, SA>();
    const uint8_t *bb = q8_b<TM, SB>();
#pragma unroll
    for (int c = 0; c < T::NBK; ++c) {
        const int row = bcol[c] + lr;
        const uint4 v = *(const uint4 *)(bb + row * kQ8BRow + (((2 * HS + lh) ^ q8_bswz(row)) << 4));
        fb[c] = int32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int m = 0; m < T::MB; ++m) {
        const int row = arow0 + m * 32 + lr;
        const uint4 v0 = *(const uint4 *)(ab + bswz(row, 4 * HS + lh));
        const uint4 v1 = *(const uint4 *)(ab + bswz(row, 4 * HS + 2 + lh));
        fa[m] = int32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
    }
}

// The scale words of a step: activation rows arow0 + 32m + lr, weight rows bcol[c] + lr.
template <int TM, int SA, int SB>
__device__ __forceinline__ void q8_read_scales(uint32_t (&sa)[BigTile<TM>::MB], uint32_t (&sb)[BigTile<TM>::NBK],
                                               const int (&bcol)[BigTile<TM>::NBK], int arow0, int lr) {
    using T = BigTile<TM>;
    const uint8_t *ab = q8_a<TM, SA>() + T::BM * kBigRow;
    const uint8_t *bb = q8_b<TM, SB>() + T::BN * kQ8BRow;
#pragma unroll
    for (int m = 0; m < T::MB; ++m) sa[m] = *(const uint32_t *)(ab + (arow0 + m * 32 + lr) * 4);
#pragma unroll
    for (int c = 0; c < T::NBK; ++c) sb[c] = *(const uint32_t *)(bb + (bcol[c] + lr) * 4);
}

// The scaled MFMAs of sub-step HS: the lane's scale byte of its 32-block is
// byte 2 HS + lh of the row's word (moved to byte 0: op_sel 0).
template <int TM, int HS>
__device__ __forceinline__ void q8_mma(floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                       const int32x8_t (&fa)[BigTile<TM>::MB], const int32x8_t (&fb)[BigTile<TM>::NBK],
                                       const uint32_t (&sa)[BigTile<TM>::MB], const uint32_t (&sb)[BigTile<TM>::NBK],
                                       int lh) {
    using T = BigTile<TM>;
    const int sh = 8 * (2 * HS + lh);
#pragma unroll
    for (int m = 0; m < T::MB; ++m)
#pragma unroll
        for (int c = 0; c < T::NBK; ++c)
            acc[m][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[c], fa[m], acc[m][c], 4, 0, 0,
                                                                         (int)(sb[c] >> sh), 0, (int)(sa[m] >> sh));
}

// Step st with activations in slot SA = st % 2 and weights in SB = st % 3.
// On entry f0 holds sub-step 0 of step st and s0 its scale words; A(st+1),
// B(st+1), B(st+2) are in flight, issued in the order B(st+1), A(st+1),
// B(st+2).  Reads sub-step 1 into f1 under the MFMAs of sub-step 0, waits for
// its own A(st+1), B(st+1) (all but the last NBX loads), passes the barrier,
// issues A(st+2) into SA and B(st+3) into SB (clamped to the last step:
// clamped loads are never read), reads sub-step 0 and the scales of step
// st+1 into f0, s1 under the MFMAs of sub-step 1, then hands s1 over to s0.
template <int TM, int SA, int SB>
__device__ __forceinline__ void q8_step(const Q8Ctx &c, floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                        int32x8_t (&fa0)[BigTile<TM>::MB], int32x8_t (&fb0)[BigTile<TM>::NBK],
                                        int32x8_t (&fa1)[BigTile<TM>::MB], int32x8_t (&fb1)[BigTile<TM>::NBK],
                                        uint32_t (&sa0)[BigTile<TM>::MB], uint32_t (&sb0)[BigTile<TM>::NBK],
                                        const int (&bcol)[BigTile<TM>::NBK], int st, int nstep, int wave, int arow0,
                                        int lane) {
    using T = BigTile<TM>;
    using Q = Q8Tile<TM>;
    const int lr = lane & 31, lh = lane >> 5;
    q8_read<TM, SA, SB, 1>(fa1, fb1, bcol, arow0, lr, lh);
    q8_mma<TM, 0>(acc, fa0, fb0, sa0, sb0, lh);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(Q::NBX));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    q8_issue_a<TM, SA>(c, min(st + 2, nstep - 1), wave);
    q8_issue_b<TM, SB>(c, min(st + 3, nstep - 1), wave);
    uint32_t sa1[T::MB], sb1[T::NBK];
    q8_read<TM, SA ^ 1, (SB + 1) % kRingB, 0>(fa0, fb0, bcol, arow0, lr, lh);
    q8_read_scales<TM, SA ^ 1, (SB + 1) % kRingB>(sa1, sb1, bcol, arow0, lr);
    q8_mma<TM, 1>(acc, fa1, fb1, sa0, sb0, lh);
    // the LDS reads spread over the first half of the sub-step's MFMAs, the
    // loads over the second half
    constexpr int NL = Q::NA + Q::NAS + Q::NBX, NR = 2 * T::MB + T::NBK + T::MB + T::NBK, NM = T::MB * T::NBK;
    constexpr int H1 = NM / 2, H2 = NM - NM / 2;
    constexpr int RPM = (NR + H1 - 1) / H1, LPM = (NL + H2 - 1) / H2;
#pragma unroll
    for (int i = 0; i < H1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);  // LDS reads
    }
#pragma unroll
    for (int i = 0; i < H2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, LPM, 0);  // direct-to-LDS loads
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
    for (int m = 0; m < T::MB; ++m) sa0[m] = sa1[m];
#pragma unroll
    for (int cc = 0; cc < T::NBK; ++cc) sb0[cc] = sb1[cc];
}

// The K loop: prologue, steps in groups of six (one turn of both slot
// cycles), and a tail of 0, 2 or 4 steps (nstep is a multiple of 4).
template <int TM>
__device__ __forceinline__ void q8_kloop(const Q8Ctx &c, floatx16_t (&acc)[BigTile<TM>::MB][BigTile<TM>::NBK],
                                         const int (&bcol)[BigTile<TM>::NBK], int nstep, int wave, int arow0,
                                         int lane) {
    using T = BigTile<TM>;
    using Q = Q8Tile<TM>;
    const int lr = lane & 31, lh = lane >> 5;
    q8_issue_a<TM, 0>(c, 0, wave);
    q8_issue_b<TM, 0>(c, 0, wave);
    q8_issue_b<TM, 1>(c, 1, wave);
    q8_issue_a<TM, 1>(c, 1, wave);
    q8_issue_b<TM, 2>(c, 2, wave);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * Q::NBX + Q::NA + Q::NAS));  // A(0) and B(0) landed
    __builtin_amdgcn_s_barrier();
    int32x8_t fa0[T::MB], fb0[T::NBK], fa1[T::MB], fb1[T::NBK];
    uint32_t sa0[T::MB], sb0[T::NBK];
    q8_read<TM, 0, 0, 0>(fa0, fb0, bcol, arow0, lr, lh);
    q8_read_scales<TM, 0, 0>(sa0, sb0, bcol, arow0, lr);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    int st = 0;
    for (; st + 6 <= nstep; st += 6) {
        q8_step<TM, 0, 0>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 0, nstep, wave, arow0, lane);
        q8_step<TM, 1, 1>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 1, nstep, wave, arow0, lane);
        q8_step<TM, 0, 2>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 2, nstep, wave, arow0, lane);
        q8_step<TM, 1, 0>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 3, nstep, wave, arow0, lane);
        q8_step<TM, 0, 1>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 4, nstep, wave, arow0, lane);
        q8_step<TM, 1, 2>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 5, nstep, wave, arow0, lane);
    }
    if (st + 2 <= nstep) {
        q8_step<TM, 0, 0>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 0, nstep, wave, arow0, lane);
        q8_step<TM, 1, 1>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 1, nstep, wave, arow0, lane);
        if (st + 4 <= nstep) {
            q8_step<TM, 0, 2>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 2, nstep, wave, arow0, lane);
            q8_step<TM, 1, 0>(c, acc, fa0, fb0, fa1, fb1, sa0, sb0, bcol, st + 3, nstep, wave, arow0, lane);
        }
    }
}

// One output tile (row tile rt, column block nb) of a grouped GEMM on MXFP8
// activations and MXFP4 weights, in mode TM.
template <int EPI, bool GROUPED, int OT, int TM>
__device__ __forceinline__ void q8_item(const GemmArgs &a, const RowTile &rt, int64_t nb, int wave, int lane) {
    using S = BigTile<TM>;
    using Q = Q8Tile<TM>;
    constexpr int MB = S::MB, NBK = S::NBK;
    constexpr int WCOLS = 32 * NBK;
    const int wm = TM == 1 ? 0 : wave >> 1;
    const int wn = TM == 1 ? wave : wave & 1;
    const int arow0 = wm * 32 * MB;
    lane = opaque(lane);
    const int64_t K = a.K;
    const int nstep = (int)(K / kQ8BK);  // a multiple of 4
    const int64_t brow0 = GROUPED ? (int64_t)rt.e * a.b_group_rows : 0;
    int bcol[NBK];
#pragma unroll
    for (int c = 0; c < NBK; ++c) {
        if constexpr (EPI == EPI_SWIGLU)
            bcol[c] = (c < NBK / 2) ? wn * (WCOLS / 2) + c * 32 : S::BN / 2 + wn * (WCOLS / 2) + (c - NBK / 2) * 32;
        else
            bcol[c] = wn * WCOLS + c * 32;
    }
    Q8Ctx c;
    // activation codes: load i of a wave fills LDS rows 8(wave NA + i) + lane / 8, at physical chunk
    // lane % 8 of the row's logical chunk (lane % 8) ^ swz(row); rows past the valid ones load zeros
    // (their results are never stored); gathered rows count from the buffer start, contiguous ones
    // from the tile's first row
    const uint8_t *a8 = (const uint8_t *)uniform_ptr(a.a_gather ? a.A8 : a.A8 + rt.p0 * K);
    const uint8_t *a8s = (const uint8_t *)uniform_ptr(a.a_gather ? a.A8s : a.A8s + rt.p0 * (K / 32));
    auto arow_of = [&](int row) -> int64_t {
        const int r = min(row, rt.mcount - 1);
        return a.a_gather ? (int64_t)a.a_gather[rt.p0 + r] : (int64_t)r;
    };
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        if (i < Q::NA) {
            const int lrow = (wave * Q::NA + i) * 8 + (lane >> 3);  // rows past the valid ones load zero codes
            c.aoff[i] = lrow < rt.mcount ? (uint32_t)(arow_of(lrow) * K + (((lane & 7) ^ swz(lrow)) << 4))
                                         : kPadRowOffset;
        } else {
            c.aoff[i] = 0;
        }
    }
    // activation scale words: load i of a wave fills rows 64 (wave + 4 i) + lane (rows past BM: padding)
#pragma unroll
    for (int i = 0; i < 2; ++i)
        c.asoff[i] = i < Q::NAS ? (uint32_t)(arow_of(64 * (wave + 4 * i) + lane) * (K / 32)) : 0;
    // weight codes: load i of a wave fills rows 16 (wave NBL + i) + lane / 4 at physical chunk lane % 4 of
    // logical chunk (lane % 4) ^ q8_bswz(row); SWIGLU rows past BN/2 are the matching up rows
    const int64_t bfirst = brow0 + ((EPI == EPI_SWIGLU) ? nb * (S::BN / 2) : nb * S::BN);
    const int64_t upskip = (EPI == EPI_SWIGLU) ? a.N - S::BN / 2 : 0;
    auto brel = [&](int row) -> int64_t { return row + (row >= S::BN / 2 ? upskip : 0); };
    const uint8_t *bcodes = (const uint8_t *)uniform_ptr((const uint8_t *)a.B + bfirst * (K / 2));
    const uint8_t *bscale = (const uint8_t *)uniform_ptr((const uint8_t *)a.B + a.b_rows_total * (K / 2) +
                                                         bfirst * (K / 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < Q::NBL) {
            const int row = (wave * Q::NBL + i) * 16 + (lane >> 2);
            c.boff[i] = (uint32_t)(brel(row) * (K / 2) + (((lane & 3) ^ q8_bswz(row)) << 4));
        } else {
            c.boff[i] = 0;
        }
    }
    c.bsoff = (uint32_t)(brel(min(wave * 64 + lane, S::BN - 1)) * (K / 32));
    c.ra = ring_rsrc(a8);
    c.ras = ring_rsrc(a8s);
    c.rb = ring_rsrc(bcodes);
    c.rbs = ring_rsrc(bscale);

    floatx16_t acc[MB][NBK];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int cc = 0; cc < NBK; ++cc)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][cc][r] = 0.f;
    q8_kloop<TM>(c, acc, bcol, nstep, wave, arow0, lane);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    big_epilogue<EPI, OT, TM>(a, rt, nb, acc, bcol, arow0, opaque(lane), 0);
}

constexpr int kXcds = 8;  // workgroup b runs on XCD b % 8 (round-robin dispatch, checked on the chip)

// Dense launches: the items of a round (one per workgroup) are cut into one
// chunk per XCD, and a chunk holds a few row tiles x several column blocks
// (row bands of kDenseBand tiles, column-major inside a band), so an XCD's
// L2 sees kDenseBand A row panels and nslot / kDenseBand B panels per round
// instead of every row tile of the round.  Returns the item's (t, nb).
constexpr int kDenseBand = 8;
__host__ __device__ inline void dense_item(uint32_t L, uint32_t ntiles, uint32_t nblocks, uint32_t &t,
                                           uint32_t &nb) {
    const uint32_t band = L / (kDenseBand * nblocks);
    const uint32_t rows = ntiles - band * kDenseBand < kDenseBand ? ntiles - band * kDenseBand : kDenseBand;
    const uint32_t w = L - band * kDenseBand * nblocks;
    nb = w / rows;
    t = band * kDenseBand + w % rows;
}

// Grouped launches (one tile mode each): tile t runs on XCD t % 8 and its
// column blocks are spread over that XCD's workgroups, so the tile's A rows
// are fetched into the XCD's L2 once and every weight block of the expert
// is read once.
template <int EPI, bool MX, bool GROUPED, int AT, int OT, int TM>
__device__ __forceinline__ void big_kernel_body(const GemmArgs &a) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nblocks = big_nblocks<EPI, TM>(a.N);
    if constexpr (GROUPED) {
        // the XCD's tiles are t = xcd + 8i; its items (i, nb) run tile-major over its workgroups
        const int ntiles = *a.ntiles;
        const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, nslot = gridDim.x / kXcds;
        const int64_t nx = ntiles > xcd ? (ntiles - xcd + kXcds - 1) / kXcds : 0;
        for (int64_t i = slot; i < nx * nblocks; i += nslot) {
            const int t = xcd + kXcds * (int)(i / nblocks);
            const int64_t nb = i % nblocks;
            RowTile rt;
            load_tile(a, true, BigTile<TM>::BM, t, rt);
            uniform_tile(rt);
            if constexpr (AT == ACT_Q8) q8_item<EPI, GROUPED, OT, TM>(a, rt, nb, wave, lane);
            else big_item<EPI, MX, GROUPED, AT, OT, TM>(a, rt, nb, 0, wave, lane);
        }
    } else {
        const int ntiles = (int)((a.M + BigTile<TM>::BM - 1) / BigTile<TM>::BM);
        const int ks = (EPI == EPI_F32 && !MX && a.ksplit > 1) ? a.ksplit : 1;
        const int64_t items = (int64_t)ntiles * nblocks * ks;
        // The plain order (item b + round * grid on workgroup b) gives every
        // XCD every row tile of a round once a round spans more than
        // kDenseBand of them; below that it already gives an XCD kDenseBand
        // rows or fewer.  K-sliced launches and grids of a partial XCD group
        // keep the plain order.
        const bool xmap = ks == 1 && gridDim.x % kXcds == 0 && (int64_t)gridDim.x > kDenseBand * nblocks;
        const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, nslot = gridDim.x / kXcds;
        for (int64_t r0 = 0; r0 < items; r0 += gridDim.x) {
            // round r0 / grid: XCD x takes items r0 + x * nslot + slot, slot = 0 .. nslot - 1
            const int64_t item = r0 + (xmap ? (int64_t)xcd * nslot + slot : (int64_t)blockIdx.x);
            if (item >= items) continue;
            int64_t t, nb;
            int ksl = 0;
            if (xmap) {
                uint32_t t32, nb32;  // a dense launch has far fewer than 2^32 items
                dense_item((uint32_t)item, (uint32_t)ntiles, (uint32_t)nblocks, t32, nb32);
                t = t32;
                nb = nb32;
            } else {
                ksl = (int)(item % ks);
                const int64_t tb = item / ks;
                t = tb / nblocks;
                nb = tb - t * nblocks;
            }
            RowTile rt;
            load_tile(a, false, BigTile<TM>::BM, (int)t, rt);
            big_item<EPI, MX, GROUPED, AT, OT, TM>(a, rt, nb, ksl, wave, lane);
        }
    }
}

template <int EPI, bool MX, bool GROUPED, int AT, int OT, int TM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_big_kernel(GemmArgs a) {
    big_kernel_body<EPI, MX, GROUPED, AT, OT, TM>(a);
}

// The wide mode: eight waves, two per SIMD (256 registers each).
template <int EPI, bool MX, bool GROUPED, int AT, int OT, int TM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_wide_kernel(GemmArgs a) {
    big_kernel_body<EPI, MX, GROUPED, AT, OT, TM>(a);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

constexpr int kStreamGrid = 4096;  // persistent grid cap of the streaming kernel
constexpr int kBigGrid = 256;      // persistent grid cap of the large-tile kernel (one per CU)

template <int MB, int NB, int EPI, bool MX, bool GROUPED, int AT, int OT>
static hipError_t run_stream(const GemmArgs &a, hipStream_t s) {
    const int64_t nblocks = (EPI == EPI_SWIGLU) ? a.N / (16 * (NB > 1 ? NB / 2 : 1)) : a.N / (16 * NB);
    const int64_t tiles = GROUPED ? a.max_tiles : (a.M + 16 * MB - 1) / (16 * MB);
    const int64_t items = tiles * nblocks * (EPI == EPI_F32 && !MX && !GROUPED && a.ksplit > 1 ? a.ksplit : 1);
    if (items <= 0) return hipSuccess;
    // each wave's K range holds whole 128-wide groups (register path) and at
    // least two 64-wide groups (LDS path)
    const int ks = (EPI == EPI_F32 && !MX && !GROUPED && a.ksplit > 1) ? a.ksplit : 1;
    if (a.K % (512 * ks)) return hipErrorInvalidValue;
    const int grid = (int)(items < kStreamGrid ? items : kStreamGrid);
    gemm_stream_kernel<MB, NB, EPI, MX, GROUPED, AT, OT><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int EPI, bool MX, bool GROUPED, int AT, int OT, int TM>
static hipError_t run_tile(const GemmArgs &a, hipStream_t s) {
    const int64_t nblocks = big_nblocks<EPI, TM>(a.N);
    const int64_t tiles = GROUPED ? a.max_tiles : (a.M + BigTile<TM>::BM - 1) / BigTile<TM>::BM;
    const int64_t ks = (EPI == EPI_F32 && !MX && !GROUPED && a.ksplit > 1) ? a.ksplit : 1;
    const int64_t items = tiles * nblocks * ks;
    if (items <= 0) return hipSuccess;
    // grouped launches assign tiles to XCDs and need whole XCD groups
    static_assert(kBigGrid % kXcds == 0, "the grid must cover whole XCD groups");
    const int grid = GROUPED ? kBigGrid : (int)(items < kBigGrid ? items : kBigGrid);
    if constexpr (BigTile<TM>::WAVES == 8)
        gemm_wide_kernel<EPI, MX, GROUPED, AT, OT, TM><<<grid, 512, 0, s>>>(a);
    else
        gemm_big_kernel<EPI, MX, GROUPED, AT, OT, TM><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

// Dense launches use 64-row tiles on the streaming kernel, grouped ones 16-row tiles.
template <int EPI, int NB, bool MX, bool GROUPED, int AT, int OT>
static hipError_t run_path(const GemmArgs &a, int path, hipStream_t s) {
    if (path == PATH_TILE) return run_tile<EPI, MX, GROUPED, AT, OT, 0>(a, s);
    if (path == PATH_HALF || path == PATH_TALL) {
        if constexpr (GROUPED) {
            if (path == PATH_HALF) return run_tile<EPI, MX, GROUPED, AT, OT, 1>(a, s);
            // the tall list (experts with 257..320 rows): wide tiles, tall ones for MXFP4
            return run_tile<EPI, MX, GROUPED, AT, OT, MX ? 2 : 3>(a, s);
        } else {
            return hipErrorInvalidValue;
        }
    }
    // MXFP4 weights on the register path: items of four 16-row weight blocks, so a lane's activation loads
    // (the same per item) serve twice the weight bytes of two-block items
    if constexpr (GROUPED) return run_stream<1, (MX && AT != ACT_Q8) ? 4 : NB, EPI, MX, GROUPED, AT, OT>(a, s);
    // Dense items re-read the batch's activation rows once per column block, which bounded the MXFP4
    // projections at small T: items of 16 rows and four weight blocks read a quarter of those bytes (their
    // weight rows, 4.25 bits a value, are re-read per 16-row tile from L2 instead); T=64: down 40 -> 24 us
    else return run_stream<MX ? 1 : 4, MX ? 4 : NB, EPI, MX, GROUPED, AT, OT>(a, s);
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
    if (at == ACT_F16_W16) {
        if (mx) return hipErrorInvalidValue;
        return run_path<EPI_SWIGLU, 2, false, true, ACT_F16_W16, ACT_F16>(a, path, s);
    }
    if (mx) {
        if (at == ACT_F16) return run_path<EPI_SWIGLU, 2, true, true, ACT_F16, ACT_F16>(a, path, s);
        return run_path<EPI_SWIGLU, 2, true, true, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (at == ACT_F16) return run_path<EPI_SWIGLU, 2, false, true, ACT_F16, ACT_F16>(a, path, s);
    return run_path<EPI_SWIGLU, 2, false, true, ACT_BF16, ACT_BF16>(a, path, s);
}

hipError_t launch_gemm2(const GemmArgs &a, int path, bool mx, int at, bool norm, hipStream_t s) {
    if (at == ACT_F16_W16) {
        if (mx) return hipErrorInvalidValue;
        if (norm) return run_path<EPI_NORM, 2, false, true, ACT_F16_W16, ACT_BF16>(a, path, s);
        return run_path<EPI_ACT, 2, false, true, ACT_F16_W16, ACT_BF16>(a, path, s);
    }
    if (norm) {
        if (mx) {
            if (at == ACT_F16) return run_path<EPI_NORM, 2, true, true, ACT_F16, ACT_BF16>(a, path, s);
            return run_path<EPI_NORM, 2, true, true, ACT_BF16, ACT_BF16>(a, path, s);
        }
        if (at == ACT_F16) return run_path<EPI_NORM, 2, false, true, ACT_F16, ACT_BF16>(a, path, s);
        return run_path<EPI_NORM, 2, false, true, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (mx) {
        if (at == ACT_F16) return run_path<EPI_ACT, 2, true, true, ACT_F16, ACT_BF16>(a, path, s);
        return run_path<EPI_ACT, 2, true, true, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (at == ACT_F16) return run_path<EPI_ACT, 2, false, true, ACT_F16, ACT_BF16>(a, path, s);
    return run_path<EPI_ACT, 2, false, true, ACT_BF16, ACT_BF16>(a, path, s);
}

hipError_t launch_gemm1_q8(const GemmArgs &a, int path, int ot, hipStream_t s) {
    if (ot == ACT_F16) return run_path<EPI_SWIGLU, 2, true, true, ACT_Q8, ACT_F16>(a, path, s);
    return run_path<EPI_SWIGLU, 2, true, true, ACT_Q8, ACT_BF16>(a, path, s);
}

hipError_t launch_gemm2_q8(const GemmArgs &a, int path, bool norm, hipStream_t s) {
    if (norm) return run_path<EPI_NORM, 2, true, true, ACT_Q8, ACT_BF16>(a, path, s);
    return run_path<EPI_ACT, 2, true, true, ACT_Q8, ACT_BF16>(a, path, s);
}

template <int EPI>
static hipError_t up_gemm(const GemmArgs &a, int path, bool mx, int at, hipStream_t s) {
    if (at == ACT_F16_W16) {
        if (mx) return hipErrorInvalidValue;
        return run_path<EPI, 1, false, false, ACT_F16_W16, ACT_BF16>(a, path, s);
    }
    if (mx) {
        if (at == ACT_F16) return run_path<EPI, 1, true, false, ACT_F16, ACT_BF16>(a, path, s);
        return run_path<EPI, 1, true, false, ACT_BF16, ACT_BF16>(a, path, s);
    }
    if (at == ACT_F16) return run_path<EPI, 1, false, false, ACT_F16, ACT_BF16>(a, path, s);
    return run_path<EPI, 1, false, false, ACT_BF16, ACT_BF16>(a, path, s);
}

hipError_t launch_up_gemm(const GemmArgs &a, int path, bool mx, int at, int epi, hipStream_t s) {
    if (epi == EPI_RESID) return up_gemm<EPI_RESID>(a, path, mx, at, s);
    if (epi == EPI_NORM) return up_gemm<EPI_NORM>(a, path, mx, at, s);
    if (epi == EPI_F32) return up_gemm<EPI_F32>(a, path, mx, at, s);
    return hipErrorInvalidValue;
}

// A batch of a few rows reads every activation row once per item: on the
// streaming kernel (16 weight rows an item) the activation bytes are four
// times the weight bytes at 64 rows, and a fp32 epilogue of 512 items holds
// two per CU.  A half-height tile takes 256 weight rows against the batch's
// rows, and K slices give every CU one tile.
hipError_t launch_dense_split(const GemmArgs &a, int at, hipStream_t s) {
    if (a.ksplit < 2 || a.M > BigTile<1>::BM || a.N % BigTile<1>::BN || a.K % (512 * (int64_t)a.ksplit) ||
        a.ldc != a.N)
        return hipErrorInvalidValue;
    if (at == ACT_F16_W16) return run_tile<EPI_F32, false, false, ACT_F16_W16, ACT_BF16, 1>(a, s);
    if (at == ACT_F16) return run_tile<EPI_F32, false, false, ACT_F16, ACT_BF16, 1>(a, s);
    return run_tile<EPI_F32, false, false, ACT_BF16, ACT_BF16, 1>(a, s);
}

// One thread per four adjacent outputs: the planes are added in slice order.
template <int EPI>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *planes, int ks, int64_t M, int64_t N,
                                                           void *C, const uint16_t *resid, const float *gate,
                                                           float *y) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // element p * N + n
    const int64_t plane = M * N;
    if (e >= plane) return;
    floatx4_t v = *(const floatx4_t *)(planes + e);
    for (int sl = 1; sl < ks; ++sl) {
        const floatx4_t w = *(const floatx4_t *)(planes + sl * plane + e);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += w[q];
    }
    if constexpr (EPI == EPI_RESID) {
        const uint2 hx = *(const uint2 *)(resid + e);
        const float4 gt = *(const float4 *)(gate + e % N);
        floatx4_t o;
        o[0] = bf16_to_f32((uint16_t)hx.x) + gt.x * v[0];
        o[1] = bf16_to_f32((uint16_t)(hx.x >> 16)) + gt.y * v[1];
        o[2] = bf16_to_f32((uint16_t)hx.y) + gt.z * v[2];
        o[3] = bf16_to_f32((uint16_t)(hx.y >> 16)) + gt.w * v[3];
        *(floatx4_t *)((float *)C + e) = o;
        if (y) *(floatx4_t *)(y + e) = v;
    } else {
        *(floatx4_t *)((float *)C + e) = v;
    }
}

hipError_t launch_split_reduce(const float *planes, int ks, int64_t M, int64_t N, int epi, void *C,
                               const uint16_t *resid, const float *gate, float *y, hipStream_t s) {
    if (ks < 1 || N % 4 || M < 0) return hipErrorInvalidValue;
    const int64_t groups = M * N / 4;
    if (groups == 0) return hipSuccess;
    const int grid = (int)((groups + 255) / 256);
    if (epi == EPI_RESID)
        split_reduce_kernel<EPI_RESID><<<grid, 256, 0, s>>>(planes, ks, M, N, C, resid, gate, y);
    else if (epi == EPI_F32)
        split_reduce_kernel<EPI_F32><<<grid, 256, 0, s>>>(planes, ks, M, N, C, resid, gate, y);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
