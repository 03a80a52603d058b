// Device-side helpers shared by the layer's HIP kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"  // ActType

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// D(16x16, fp32) += A(16x32) * B(32x16), bf16 or fp16 inputs.
// Lane l supplies A[l%16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l%16]
// (any permutation of k shared by A and B gives the same sum) and receives
// D[4*(l/16) + r][l%16] in element r.  ACT_Q8 operands are decoded to bf16
// before they reach an MFMA of this shape.
template <int AT>
__device__ __forceinline__ floatx4_t mfma16x16x32(uint4 a, uint4 b, floatx4_t c) {
    if constexpr (AT != ACT_BF16 && AT != ACT_Q8)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 32x32x16 MFMA: lane l supplies row l%32 of A and column l%32 of B at
// k = 8*(l/32) .. +7; it receives D[8*(r/4) + 4*(l/32) + r%4][l%32] in
// register r.  One wave per SIMD sustains close to the peak rate with this
// shape (the 16x16x32 one needs two waves per SIMD for that).
template <int AT>
__device__ __forceinline__ floatx16_t mfma32x32x16(uint4 a, uint4 b, floatx16_t c) {
    if constexpr (AT != ACT_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// fp32 -> activation bits (round to nearest even; fp16 overflows to inf).
template <int AT>
__device__ __forceinline__ uint16_t f32_to_act(float f) {
    static_assert(AT == ACT_BF16 || AT == ACT_F16, "a storage type");
    if constexpr (AT == ACT_F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
    else return f32_to_bf16(f);
}

template <int AT>
__device__ __forceinline__ float act_to_f32(uint16_t b) {
    static_assert(AT == ACT_BF16 || AT == ACT_F16, "a storage type");
    if constexpr (AT == ACT_F16) return (float)__builtin_bit_cast(_Float16, b);
    else return bf16_to_f32(b);
}

// Eight bf16 -> eight fp16, rounded to nearest even.  Exact for |w| in
// [2^-17, 65504]: a bf16 value has 8 significant bits and fp16 11, so
// nothing is rounded in that range; smaller values round to an fp16
// subnormal, larger ones overflow to inf.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
    const float lo = __uint_as_float(v << 16), hi = __uint_as_float(v & 0xffff0000u);
    const f16x2_t r = {(_Float16)lo, (_Float16)hi};  // one v_cvt_pk_f16_f32
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
    return make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w));
}

// Weight operand in the MFMA type: bf16 weights pass through (bf16 GEMM)
// or are converted to fp16; fp16 weights pass through.
template <int AT>
__device__ __forceinline__ uint4 weight_bf16_as(uint4 v) {
    if constexpr (AT == ACT_F16) return bf16x8_to_f16x8(v);
    else return v;
}

// Eight E2M1 codes (one dword, low nibble first) times 2^(E-127) -> eight
// bf16 or fp16 (exact whenever the product is representable).
template <int AT>
__device__ __forceinline__ uint4 mxfp4x8_to_act(uint32_t codes, uint32_t e8m0) {
    static_assert(AT == ACT_BF16 || AT == ACT_F16 || AT == ACT_Q8, "MXFP4 weights are decoded to bf16 or fp16");
    float scale = e8m0 ? __uint_as_float(e8m0 << 23) : __uint_as_float(0x00400000u);
    uint4 r;
    if constexpr (AT == ACT_F16) {
        r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 0));
        r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 1));
        r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 2));
        r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 3));
    } else {
        r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
        r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
        r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
        r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
    }
    return r;
}

// ---------------------------------------------------------------------------
// MXFP8 activations (OCP Microscaling Formats (MX) v1.0, MXFP8 with E4M3
// elements): 32 consecutive values along K share one E8M0 scale 2^X.
// ---------------------------------------------------------------------------

// E4M3 code of w (an exact fp32 value, |w| < 2^9): nearest E4M3 value, ties
// to even, magnitudes from 448 (the largest finite E4M3 value) up clamped to
// 448.  Normal results (|w| >= 2^-6) keep the top 3 mantissa bits after a
// round-to-nearest-even carry on the fp32 bits (a carry into the exponent is
// the next binade); below 2^-6 the E4M3 values are the multiples of 2^-9, so
// the code is w * 2^9 rounded to an integer (8 is the code of 2^-6).
__device__ __forceinline__ uint32_t e4m3_code(float w) {
    const uint32_t b = __float_as_uint(w);
    const uint32_t sgn = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7fffffffu;
    uint32_t c;
    if (a >= 0x43e00000u) c = 0x7eu;  // 448
    else if (a >= 0x3c800000u) c = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    else c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    return sgn | c;
}

// The shared exponent of a block from its largest magnitude: X =
// floor(log2 amax) - 8, clamped to [-127, 127]; returned as the E8M0 code
// X + 127 (0 for an all-zero block).  amax is a finite fp32 value.
__device__ __forceinline__ uint32_t mx8_scale_code(float amax) {
    const uint32_t e = __float_as_uint(amax) >> 23;  // biased exponent (amax >= 0)
    if (e == 0) return 0u;                           // zero (or an fp32 subnormal): the smallest scale
    const int x = (int)e - 127 - 8;
    return (uint32_t)(x < -127 ? 0 : x + 127);
}

// 2^-X for an E8M0 code X + 127 in 0..246 (the codes the quantizer makes:
// X <= 119 for a finite fp32 block maximum), a normal fp32 value.
__device__ __forceinline__ float mx8_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// 2^(E-127) as an fp32 value (E = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t e8m0) {
    return e8m0 ? __uint_as_float(e8m0 << 23) : __uint_as_float(0x00400000u);
}

// Sixteen E4M3 codes (one uint4, lowest byte first) times 2^(E-127) -> sixteen
// bf16 (two uint4), exact: an E4M3 value has 4 significant bits.
__device__ __forceinline__ void mxfp8x16_to_bf16(uint4 codes, uint32_t e8m0, uint4 &lo, uint4 &hi) {
    const float sc = e8m0_value(e8m0);
#define MOE_CV8(w, upper) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), sc, (upper)))
    lo = make_uint4(MOE_CV8(codes.x, false), MOE_CV8(codes.x, true), MOE_CV8(codes.y, false), MOE_CV8(codes.y, true));
    hi = make_uint4(MOE_CV8(codes.z, false), MOE_CV8(codes.z, true), MOE_CV8(codes.w, false), MOE_CV8(codes.w, true));
#undef MOE_CV8
}

// silu(t) = t / (1 + e^-t): `silu` with the accurate exponential and an
// IEEE division (the fp32 path), `silu_fast` with the hardware exponential
// (v_exp_f32 on -t log2 e) and reciprocal (v_rcp_f32), relative error about
// 1e-6, far below the 16-bit rounding of the GEMM epilogues' stored results
// (2^-11 for fp16); both give -0 as t -> -inf, t as t -> +inf, NaN for NaN.
__device__ __forceinline__ float silu(float t) { return t / (1.0f + expf(-t)); }
__device__ __forceinline__ float silu_fast(float t) { return t * __builtin_amdgcn_rcpf(1.0f + __expf(-t)); }

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

}  // namespace moe
