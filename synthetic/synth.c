/*
 * Seeded synthetic inputs for the latent MoE layer: weights, activations,
 * gains and the router bias.  This module is shared by the CPU oracle's tests
 * and by the GPU tests and benchmark; it holds none of the layer's arithmetic
 * (no GEMM, norm, routing or combine), only the input recipes.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of
 * J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11.  Each tensor draws from its own key,
 * derived from (seed, tensor name), and element i of the tensor uses counter
 * i/4 and output word i%4, so any slice of any tensor can be produced on its
 * own, in any order, by any number of threads, with identical results.
 *
 * Normals: the Box-Muller transform (G. E. P. Box, M. E. Muller, "A note on
 * the generation of random normal deviates", Ann. Math. Stat. 29, 1958) on
 * pairs of 24-bit uniforms, in single precision.
 *
 * Stored dtypes: bf16 by round-to-nearest-even of the fp32 draw; MXFP4 per
 * the OCP Microscaling Formats (MX) v1.0 specification: blocks of 32
 * consecutive elements along a row share one E8M0 scale X = 2^(floor(log2
 * amax) - 2); each element is v / X rounded to nearest-even on the E2M1 grid
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}, saturating at 6.
 */
#define _GNU_SOURCE /* sincosf */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

/* Philox4x32 with 10 rounds: out = philox(counter, key). */
static inline void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(PHILOX_M0, c0, &hi0, &lo0);
        mulhilo32(PHILOX_M1, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    philox4x32_10(ctr, key, out);
}

/* Key of a tensor: FNV-1a 64 of its name, mixed with the seed. */
void synth_key(uint64_t seed, const char *name, uint32_t key[2]) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (const unsigned char *p = (const unsigned char *)name; *p; ++p) {
        h ^= *p;
        h *= 0x100000001b3ull;
    }
    h ^= seed * 0x9E3779B97F4A7C15ull;
    key[0] = (uint32_t)h;
    key[1] = (uint32_t)(h >> 32);
}

static inline float u24_open(uint32_t w) { /* (0,1), never 0 */
    return ((float)(w >> 8) + 0.5f) * (1.0f / 16777216.0f);
}
static inline float u24_closed_open(uint32_t w) { /* [0,1) */
    return (float)(w >> 8) * (1.0f / 16777216.0f);
}

/* Four normals from one Philox block, by Box-Muller on (w0,w1) and (w2,w3). */
static inline void normals4(const uint32_t key[2], uint64_t blk, float z[4]) {
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
    uint32_t w[4];
    philox4x32_10(ctr, key, w);
    const float two_pi = 6.28318530717958647692f;
    for (int p = 0; p < 2; ++p) {
        float u1 = u24_open(w[2 * p]);
        float u2 = u24_closed_open(w[2 * p + 1]);
        float r = sqrtf(-2.0f * logf(u1));
        float s, c;
        sincosf(two_pi * u2, &s, &c);
        z[2 * p] = r * c;
        z[2 * p + 1] = r * s;
    }
}

/* Normal draws of elements [start, start+count) of a tensor, times std. */
void synth_normal_f32(uint64_t seed, const char *name, uint64_t start, uint64_t count, float std,
                      float *out) {
    uint32_t key[2];
    synth_key(seed, name, key);
    int64_t b0 = (int64_t)(start / 4), b1 = (int64_t)((start + count + 3) / 4);
#pragma omp parallel for schedule(static)
    for (int64_t b = b0; b < b1; ++b) {
        float z[4];
        normals4(key, (uint64_t)b, z);
        for (int j = 0; j < 4; ++j) {
            uint64_t i = (uint64_t)b * 4 + j;
            if (i >= start && i < start + count) out[i - start] = z[j] * std;
        }
    }
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void synth_f32_to_bf16(const float *in, uint16_t *out, uint64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* Normal draws rounded to bf16 (bit patterns). */
void synth_normal_bf16(uint64_t seed, const char *name, uint64_t start, uint64_t count, float std,
                       uint16_t *out) {
    uint32_t key[2];
    synth_key(seed, name, key);
    int64_t b0 = (int64_t)(start / 4), b1 = (int64_t)((start + count + 3) / 4);
#pragma omp parallel for schedule(static)
    for (int64_t b = b0; b < b1; ++b) {
        float z[4];
        normals4(key, (uint64_t)b, z);
        for (int j = 0; j < 4; ++j) {
            uint64_t i = (uint64_t)b * 4 + j;
            if (i >= start && i < start + count) out[i - start] = f32_to_bf16_rne(z[j] * std);
        }
    }
}

/* Uniform [lo, hi) draws (fp32) of elements [start, start+count). */
void synth_uniform_f32(uint64_t seed, const char *name, uint64_t start, uint64_t count, float lo,
                       float hi, float *out) {
    uint32_t key[2];
    synth_key(seed, name, key);
    int64_t b0 = (int64_t)(start / 4), b1 = (int64_t)((start + count + 3) / 4);
#pragma omp parallel for schedule(static)
    for (int64_t b = b0; b < b1; ++b) {
        uint32_t ctr[4] = {(uint32_t)b, (uint32_t)((uint64_t)b >> 32), 0u, 0u}, w[4];
        philox4x32_10(ctr, key, w);
        for (int j = 0; j < 4; ++j) {
            uint64_t i = (uint64_t)b * 4 + j;
            if (i >= start && i < start + count) out[i - start] = lo + (hi - lo) * u24_closed_open(w[j]);
        }
    }
}

/* ---- MXFP4 (OCP MX v1.0): E2M1 elements, one E8M0 scale per 32 along K ---- */

static inline uint8_t e2m1_rne(float a) { /* a = |v|/X >= 0; returns the 3-bit magnitude code */
    if (a <= 0.25f) return 0;  /* 0   */
    if (a < 0.75f) return 1;   /* 0.5 */
    if (a <= 1.25f) return 2;  /* 1   */
    if (a < 1.75f) return 3;   /* 1.5 */
    if (a <= 2.5f) return 4;   /* 2   */
    if (a < 3.5f) return 5;    /* 3   */
    if (a <= 5.0f) return 6;   /* 4   */
    return 7;                  /* 6 (saturating) */
}

/* Quantise one block of 32 values: writes 16 packed bytes (low nibble = even
 * element) and returns the E8M0 scale byte. */
static uint8_t quant_block32(const float *v, uint8_t *packed) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    int e;
    if (amax == 0.0f) {
        e = -127;
    } else {
        int ex;
        frexpf(amax, &ex);      /* amax = m * 2^ex, m in [0.5,1) => floor(log2 amax) = ex-1 */
        e = (ex - 1) - 2;       /* largest E2M1 power is 2^2 */
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    float inv = ldexpf(1.0f, -e);
    for (int i = 0; i < 32; i += 2) {
        uint8_t q[2];
        for (int h = 0; h < 2; ++h) {
            float x = v[i + h] * inv;
            uint8_t m = e2m1_rne(fabsf(x));
            q[h] = (uint8_t)((m != 0 && x < 0.0f) ? (m | 8u) : m);
        }
        packed[i / 2] = (uint8_t)(q[0] | (q[1] << 4));
    }
    return (uint8_t)(e + 127);
}

void synth_mxfp4_quantize(const float *v, int64_t rows, int64_t K, uint8_t *packed, uint8_t *scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / 32; ++b)
            scales[r * (K / 32) + b] = quant_block32(v + r * K + b * 32, packed + r * (K / 2) + b * 16);
}

/* Rows [row0, row0+nrows) of a [rows][K] tensor of N(0,std) draws (the same
 * draws synth_normal_f32 gives), rounded to bf16 (bf16: [nrows][K], may be
 * NULL) and/or quantised to MXFP4 (packed: [nrows][K/2] and scales:
 * [nrows][K/32], may be NULL).  K must be a multiple of 32. */
void synth_normal_rows(uint64_t seed, const char *name, int64_t row0, int64_t nrows, int64_t K,
                       float std, uint16_t *bf16, uint8_t *packed, uint8_t *scales) {
    uint32_t key[2];
    synth_key(seed, name, key);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        float row[32];
        for (int64_t b = 0; b < K / 32; ++b) {
            uint64_t base = (uint64_t)(row0 + r) * (uint64_t)K + (uint64_t)b * 32;
            for (int q = 0; q < 8; ++q) {
                float z[4];
                normals4(key, base / 4 + q, z);
                for (int j = 0; j < 4; ++j) row[q * 4 + j] = z[j] * std;
            }
            if (bf16)
                for (int j = 0; j < 32; ++j) bf16[r * K + b * 32 + j] = f32_to_bf16_rne(row[j]);
            if (packed)
                scales[r * (K / 32) + b] = quant_block32(row, packed + r * (K / 2) + b * 16);
        }
    }
}
