/*
 * CPU ORACLE for the latent sparse mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU path: it is a plain, slow, fp64
 * evaluation of the definitions, written to be checked by eye against the
 * pages it cites:
 *
 *  [Gates]    flozi.net, "Muse Spark Open: Norm-Preserving Gates Are Not a
 *             Norm Guarantee" (sections "Two normalization orders implement
 *             different functions", "Latent experts: normalization happens
 *             before the weighted sum", "What this means for serving and
 *             kernel work").
 *  [Shazeer]  bobbyburns.tech, "816 billion parameters, and only 42 billion
 *             show up for each token" (section "The math": "Setup" with the
 *             equation y = sum_i G(x)_i E_i(x), and "The gate" with
 *             G = Softmax(KeepTopK(H, k)) and its worked example).
 *  [FactSheet] archdb.vladsavinov.com, "Muse-Spark-Open-816B-A42B" (fields
 *             FFN activation SwiGLU, no FFN bias, no GLU clamp,
 *             routed_scaling_factor 1, latent width 4,096, gating function
 *             sigmoid, block norm RMSNorm with a 1+w gain and epsilon 1e-5,
 *             residual design alpha*residual + beta*h).
 *
 * Precision: every sum, product and transcendental is fp64.  Values are
 * rounded only where the method itself stores them in a narrower type:
 *  - router logits are FP32 ([Gates] "FP32 router logits"; the router is an
 *    FP32 module), so top-k selection is decided on fp32-rounded logits and
 *    an fp32 add of the selection bias;
 *  - a norm returns its input dtype ([Gates], serving section), and the
 *    input-scaled norm rounds the scaled vector to the input dtype before
 *    its reduction ([Gates], normalization-orders section);
 *  - with act_quant = MXFP8 (a mode of this build, not of the pages) the
 *    inputs of the two expert GEMMs (the latent z and the SwiGLU output)
 *    are the stored intermediates (rounded to the intermediate dtype)
 *    quantized to MXFP8 per OCP MX v1.0, since that is what those GEMMs
 *    multiply in that mode;
 *  - optional "mirror" mode additionally rounds the latent z, the SwiGLU
 *    output and the mixture m to an intermediate dtype (bf16 or fp16), the
 *    way a device stores them between GEMMs (a diagnostic, not a bar).
 *
 * Parity pins: see the oracle's tests.  Unpinned readings (each also listed
 * in the design notes): the epsilon placement x*(mean(x^2)+eps)^-1/2, the
 * MXFP4 quantiser choice (the oracle consumes already-quantised bits), the
 * I_gamma double-rounding corner.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_MXFP4 = 2, ORC_F16 = 3, ORC_MXFP8 = 4 };
enum { ORC_NORM_NONE = 0, ORC_NORM_CENTERED = 1, ORC_NORM_INPUT_SCALED = 2 };
enum { ORC_RELU = 0, ORC_SWIGLU = 1 };
enum { ORC_RES_NONE = 0, ORC_RES_LINEAR = 1, ORC_RES_MUSE = 2 };
enum { ORC_ROUTER_SOFTMAX = 0, ORC_ROUTER_SIGMOID = 1 };
enum { ORC_AQ_NONE = 0, ORC_AQ_MXFP8 = 1 };

typedef struct {
    int64_t d, L, n, k, F; /* L == 0: no latent projection, experts read u directly */
    int32_t kind;          /* ORC_RELU: W2 relu(W1 u); ORC_SWIGLU: W2 (silu(Wg z) * (Wu z)) */
    int32_t act;           /* stored dtype of x (and of the norms' outputs): F32 or BF16 */
    int32_t wdt;           /* dtype of down/up/expert weights: F32, BF16, MXFP4 */
    int32_t rdt;           /* dtype of the router weight: F32 or BF16 */
    int32_t in_norm;       /* norm applied to x before router and down-projection */
    int32_t ex_norm;       /* norm applied to every expert output before mixing */
    int32_t res_gate;      /* ORC_RES_NONE: out = b; LINEAR: out = h + g*b; MUSE: alpha*h + beta*b
                              (h = x, b = the branch output after the optional output norm) */
    int32_t bias_in_weights; /* softmax router: 0 = bias only changes selection */
    double eps_in, eps_ex;
    int32_t mirror;        /* 1: round z, a and m to the intermediate dtype (debug aid) */
    int32_t interm;        /* intermediate dtype of mirror mode: ORC_BF16 or ORC_F16 */
    int32_t router_fn;     /* ORC_ROUTER_SOFTMAX or ORC_ROUTER_SIGMOID */
    double out_mult;       /* sigmoid router: logit multiplier before the sigmoid */
    double rsf;            /* sigmoid router: routed scaling factor of the weights */
    int32_t lat_norm;      /* norm of the latent P_down u before the experts (C_pre) */
    int32_t out_norm;      /* norm of the branch output P_up m (the FFN output norm) */
    double eps_lat, eps_out;
    double tau, floor_;    /* ORC_RES_MUSE: temperature and floor of the residual gate */
    int32_t act_quant;     /* ORC_AQ_MXFP8: the expert GEMMs read MXFP8 activations (the latent z and
                              the SwiGLU output, stored in the intermediate dtype, then quantized) */
} orc_desc;

typedef struct {
    const void *x;        /* [T][d], act */
    const void *router_w; /* [n][d], rdt */
    const void *down_w;   /* [L][d], wdt */
    const void *w1;       /* SwiGLU: [n][2F][L] (gate rows then up rows); ReLU: [n][F][d] */
    const void *w2;       /* SwiGLU: [n][L][F]; ReLU: [n][d][F] */
    const void *up_w;     /* [d][L] */
    const float *bias;    /* [n] or NULL */
    const float *gamma_in; /* [d] or NULL */
    const float *gamma_ex; /* [L] (ReLU: [d]) or NULL */
    const float *gate;    /* [d] or NULL */
    const float *gamma_lat; /* [L] or NULL */
    const float *gamma_out; /* [d] or NULL */
} orc_tensors;

/* ------------------------------------------------------------------ */
/* Stored-type decoding and rounding                                   */
/* ------------------------------------------------------------------ */

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest bf16 value (ties to even), returned as a
 * double.  Done in two exact steps: the double is first rounded to the
 * nearest float only when that cannot cause a double-rounding error;
 * otherwise the bf16 grid is applied directly to the double. */
static double round_to_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    frexp(v, &e);            /* |v| in [2^(e-1), 2^e) */
    if (e - 1 < -126) e = -125; /* below the normal range the spacing is fixed */
    /* bf16 keeps 8 significant bits: spacing 2^(e-1-7) */
    double q = ldexp(1.0, e - 1 - 7);
    double r = v / q;        /* exact: power-of-two scaling */
    double fl = floor(r);
    double diff = r - fl;
    double res;
    if (diff > 0.5) res = fl + 1.0;
    else if (diff < 0.5) res = fl;
    else res = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    return res * q;
}

static double round_to_f32(double v) { return (double)(float)v; }

/* Round a double to the nearest IEEE half value (ties to even): 11
 * significant bits, spacing 2^-24 below 2^-14, overflow to infinity past
 * the largest finite value 65504. */
static double round_to_f16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    frexp(v, &e);
    if (e - 1 < -14) e = -13;
    double q = ldexp(1.0, e - 1 - 10);
    double r = v / q, fl = floor(r), diff = r - fl, res;
    if (diff > 0.5) res = fl + 1.0;
    else if (diff < 0.5) res = fl;
    else res = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    res *= q;
    if (fabs(res) > 65504.0) return res > 0 ? INFINITY : -INFINITY;
    return res;
}

static double round_act(int act, double v) {
    if (act == ORC_BF16) return round_to_bf16(v);
    if (act == ORC_F16) return round_to_f16(v);
    return round_to_f32(v);
}

/* OCP MX v1.0: E2M1 element = (-1)^s * 2^(E-1) * (1 + m/2), E in 1..3; E=0: m/2. */
static double e2m1_value(unsigned code) {
    unsigned s = (code >> 3) & 1u, E = (code >> 1) & 3u, m = code & 1u;
    double mag = (E == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)E - 1);
    return s ? -mag : mag;
}

/* E8M0 scale = 2^(E-127). */
static double e8m0_value(unsigned E) { return ldexp(1.0, (int)E - 127); }

/* ------------------------------------------------------------------ */
/* MXFP8 activations (OCP Microscaling Formats (MX) v1.0, MXFP8 with   */
/* E4M3 elements).  A block of 32 consecutive values along the         */
/* reduction dimension shares one power-of-two scale 2^X, with         */
/* X = floor(log2(max |v|)) - 8 (8 is the largest exponent of an E4M3  */
/* element); each value becomes v / 2^X rounded to the nearest E4M3    */
/* value, ties to even, a magnitude beyond the largest finite E4M3     */
/* value (448) clamped to it.  An all-zero block keeps the smallest    */
/* scale (E8M0 code 0) and zero elements.                              */
/* ------------------------------------------------------------------ */

/* Nearest E4M3 value to v (ties to even), clamped to [-448, 448].  E4M3
 * has 3 mantissa bits, normal exponents -6..8 and subnormals of spacing
 * 2^-9. */
static double round_to_e4m3(double v) {
    if (v == 0.0 || isnan(v)) return v;
    double a = fabs(v);
    if (a >= 448.0) return copysign(448.0, v);
    int e;
    frexp(a, &e);            /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -6) ex = -6;    /* below the normal range the spacing is fixed */
    double q = ldexp(1.0, ex - 3);
    double r = a / q, fl = floor(r), diff = r - fl, res;
    if (diff > 0.5) res = fl + 1.0;
    else if (diff < 0.5) res = fl;
    else res = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    res *= q;
    if (res > 448.0) res = 448.0;
    return copysign(res, v);
}

/* One MX block of n (<= 32) values quantized in place to its dequantized
 * values q_i * 2^X; returns X (-127 for an all-zero block). */
static int mxfp8_block(double *v, int64_t n) {
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) {
        for (int64_t i = 0; i < n; ++i) v[i] = 0.0;
        return -127;
    }
    int e;
    frexp(amax, &e);         /* floor(log2(amax)) = e - 1 */
    int X = e - 1 - 8;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    double sc = ldexp(1.0, X);
    for (int64_t i = 0; i < n; ++i) v[i] = round_to_e4m3(v[i] / sc) * sc;
    return X;
}

/* v[0..n) (n a multiple of 32) quantized block by block to MXFP8, in place;
 * X[b] (may be NULL) receives the scale exponent of block b. */
void orc_mxfp8_quantize(double *v, int64_t n, int32_t *X) {
    for (int64_t b = 0; b * 32 < n; ++b) {
        int x = mxfp8_block(v + b * 32, 32);
        if (X) X[b] = x;
    }
}

/* The value an expert GEMM reads under MXFP8 activations: the stored
 * intermediate (rounded to the intermediate dtype), then quantized. */
static void quantize_activations(const orc_desc *d, double *v, int64_t n) {
    if (d->act_quant != ORC_AQ_MXFP8) return;
    for (int64_t i = 0; i < n; ++i) v[i] = round_act(d->interm, v[i]);
    orc_mxfp8_quantize(v, n, NULL);
}

/* OCP FP8 E4M3 element: (-1)^s * 2^(E-7) * (1 + m/8) for E in 1..15, (-1)^s *
 * 2^-6 * m/8 for E = 0; S.1111.111 is NaN (there are no infinities). */
static double e4m3_value(unsigned code) {
    unsigned s = (code >> 7) & 1u, E = (code >> 3) & 15u, m = code & 7u;
    if (E == 15 && m == 7) return NAN;
    double mag = (E == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)E - 7);
    return s ? -mag : mag;
}

/* Row r (of a [rows][K] matrix) decoded to doubles.  MXFP4 matrices are one
 * buffer: packed nibbles [rows][K/2] (low nibble = even element), then E8M0
 * scales [rows][K/32]; MXFP8 matrices: E4M3 codes [rows][K], then E8M0 scales
 * [rows][K/32]. */
static void load_row(const void *base, int dt, int64_t rows, int64_t K, int64_t r, double *out) {
    if (dt == ORC_F32) {
        const float *p = (const float *)base + r * K;
        for (int64_t c = 0; c < K; ++c) out[c] = (double)p[c];
    } else if (dt == ORC_BF16) {
        const uint16_t *p = (const uint16_t *)base + r * K;
        for (int64_t c = 0; c < K; ++c) out[c] = bf16_bits_to_double(p[c]);
    } else if (dt == ORC_MXFP8) {
        /* the element values by code, from the definition above (a lookup, not a new formula) */
        double val[256];
        for (unsigned q = 0; q < 256; ++q) val[q] = e4m3_value(q);
        const uint8_t *cd = (const uint8_t *)base + r * K;
        const uint8_t *sc = (const uint8_t *)base + rows * K + r * (K / 32);
        for (int64_t b = 0; b < K / 32; ++b) {
            const double scale = e8m0_value(sc[b]);
            for (int64_t c = 32 * b; c < 32 * b + 32; ++c) out[c] = val[cd[c]] * scale;
        }
    } else {
        double val[16];
        for (unsigned q = 0; q < 16; ++q) val[q] = e2m1_value(q);
        const uint8_t *nib = (const uint8_t *)base + r * (K / 2);
        const uint8_t *sc = (const uint8_t *)base + rows * (K / 2) + r * (K / 32);
        for (int64_t b = 0; b < K / 32; ++b) {
            const double scale = e8m0_value(sc[b]);
            for (int64_t c = 32 * b; c < 32 * b + 32; ++c) {
                unsigned code = (nib[c / 2] >> (4 * (c & 1))) & 15u;
                out[c] = val[code] * scale;
            }
        }
    }
}

static double dot(const double *a, const double *b, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* out[r] = sum_c W[row0 + r][c] * v[c] for r < nout: a plain matrix-vector
 * product, rows computed independently (in parallel over rows). */
static void matvec(const void *W, int dt, int64_t rows, int64_t K, int64_t row0, int64_t nout,
                   const double *v, double *out) {
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < nout; ++r) {
            load_row(W, dt, rows, K, row0 + r, row);
            out[r] = dot(row, v, K);
        }
        free(row);
    }
}

/* ------------------------------------------------------------------ */
/* RMS norms ([Gates], "Two normalization orders ...")                 */
/* R_eps(x) = x * (mean(x^2) + eps)^(-1/2); D_gamma = diag(1 + gamma).  */
/* ------------------------------------------------------------------ */

/* C_gamma(x) = D_gamma R_eps(x): output-scaled ("centered" = 1+gamma gain). */
void orc_rms_centered(const double *x, const float *gamma, int64_t D, double eps, double *out) {
    double ss = 0.0;
    for (int64_t i = 0; i < D; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (int64_t i = 0; i < D; ++i) out[i] = (1.0 + (gamma ? (double)gamma[i] : 0.0)) * x[i] * inv;
}

/* I_gamma(x) = R_eps(D_gamma x), with the scaled vector D_gamma x rounded to
 * the input dtype before the reduction (act: ORC_F32 / ORC_BF16; -1 = no
 * rounding, the real-arithmetic form). */
void orc_rms_input_scaled(const double *x, const float *gamma, int64_t D, double eps, int act,
                          double *out) {
    double ss = 0.0;
    for (int64_t i = 0; i < D; ++i) {
        double s = (1.0 + (gamma ? (double)gamma[i] : 0.0)) * x[i];
        if (act >= 0) s = round_act(act, s);
        out[i] = s;
        ss += s * s;
    }
    double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (int64_t i = 0; i < D; ++i) out[i] *= inv;
}

static void apply_norm(int kind, const double *x, const float *gamma, int64_t D, double eps, int act,
                       double *out) {
    if (kind == ORC_NORM_CENTERED) orc_rms_centered(x, gamma, D, eps, out);
    else if (kind == ORC_NORM_INPUT_SCALED) orc_rms_input_scaled(x, gamma, D, eps, act, out);
    else memcpy(out, x, sizeof(double) * (size_t)D);
}

/* ------------------------------------------------------------------ */
/* Gate ([Shazeer], "The gate"): G = Softmax(KeepTopK(H, k)).          */
/* ------------------------------------------------------------------ */

/* Selection: the k largest scores, largest first; equal scores keep the
 * lower expert id first.  margin = k-th score minus (k+1)-th score. */
void orc_topk(const double *score, int64_t n, int64_t k, int32_t *idx, double *margin) {
    char *taken = (char *)calloc((size_t)n, 1);
    double kth = 0.0;
    for (int64_t j = 0; j < k; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < n; ++e)
            if (!taken[e] && (best < 0 || score[e] > score[best])) best = e;
        taken[best] = 1;
        idx[j] = (int32_t)best;
        kth = score[best];
    }
    if (margin) {
        int64_t nxt = -1;
        for (int64_t e = 0; e < n; ++e)
            if (!taken[e] && (nxt < 0 || score[e] > score[nxt])) nxt = e;
        *margin = (nxt < 0) ? INFINITY : kth - score[nxt];
    }
    free(taken);
}

/* Softmax over the kept entries of H (every other entry is -inf, weight 0):
 * w_j = exp(H[idx_j]) / sum_j' exp(H[idx_j']), computed relative to the
 * largest kept value. */
void orc_softmax_kept(const double *H, const int32_t *idx, int64_t k, double *w) {
    double mx = -INFINITY;
    for (int64_t j = 0; j < k; ++j) if (H[idx[j]] > mx) mx = H[idx[j]];
    double s = 0.0;
    for (int64_t j = 0; j < k; ++j) { w[j] = exp(H[idx[j]] - mx); s += w[j]; }
    for (int64_t j = 0; j < k; ++j) w[j] /= s;
}

/* Dense gate vector G (length n): the softmax weights at the kept experts,
 * exactly 0 elsewhere. */
void orc_gate_dense(const double *H, int64_t n, int64_t k, double *G) {
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double *w = (double *)malloc(sizeof(double) * (size_t)k);
    orc_topk(H, n, k, idx, NULL);
    orc_softmax_kept(H, idx, k, w);
    for (int64_t e = 0; e < n; ++e) G[e] = 0.0;
    for (int64_t j = 0; j < k; ++j) G[idx[j]] = w[j];
    free(idx);
    free(w);
}

/* ------------------------------------------------------------------ */
/* One token through the layer                                         */
/* ------------------------------------------------------------------ */

static double load_x(const orc_desc *d, const void *x, int64_t t, int64_t i) {
    if (d->act == ORC_BF16) return bf16_bits_to_double(((const uint16_t *)x)[t * d->d + i]);
    return (double)((const float *)x)[t * d->d + i];
}

/* u = branch input: x, or its input norm, returned in the input dtype. */
static void branch_input(const orc_desc *d, const orc_tensors *w, int64_t t, double *h, double *u) {
    for (int64_t i = 0; i < d->d; ++i) h[i] = load_x(d, w->x, t, i);
    if (d->in_norm == ORC_NORM_NONE) {
        memcpy(u, h, sizeof(double) * (size_t)d->d);
        return;
    }
    apply_norm(d->in_norm, h, w->gamma_in, d->d, d->eps_in, d->act, u);
    for (int64_t i = 0; i < d->d; ++i) u[i] = round_act(d->act, u[i]);
}

/* ------------------------------------------------------------------ */
/* Router scores and weights.                                          */
/*  softmax ([Shazeer] "The gate"; [Gates] latent-experts section for  */
/*  the FP32 logits and the selection-only bias): selection score      */
/*  s = fp32(l + b), weights = softmax over the kept logits (over the  */
/*  kept s when bias_in_weights).                                      */
/*  sigmoid ([Gates] latent-experts section; [FactSheet] gating        */
/*  function): sigma = fp32(sigmoid(fp32(l * output_multiplier))), the */
/*  router being an FP32 module; selection score s = fp32(sigma + b);  */
/*  weights = the kept sigma divided by (their sum + 1e-15), times the */
/*  routed scaling factor.                                             */
/* ------------------------------------------------------------------ */

/* From fp32 logits l[n] and bias b[n] (or NULL): selection scores sel[n]
 * and the values H[n] the weights are computed from. */
void orc_router_scores(const orc_desc *d, const float *l, const float *bias, double *sel, double *H) {
    for (int64_t e = 0; e < d->n; ++e) {
        float b = bias ? bias[e] : 0.0f;
        if (d->router_fn == ORC_ROUTER_SIGMOID) {
            float v = (float)((double)l[e] * d->out_mult);           /* fp32 product */
            float sg = (float)(1.0 / (1.0 + exp(-(double)v)));       /* fp32 sigmoid */
            sel[e] = (double)(bias ? sg + b : sg);                  /* fp32 add */
            H[e] = (double)sg;
        } else {
            float sf = bias ? l[e] + b : l[e];                      /* fp32 add */
            sel[e] = (double)sf;
            H[e] = d->bias_in_weights ? (double)sf : (double)l[e];
        }
    }
}

/* Weights of the kept experts idx[0..k) from the values H. */
void orc_router_weights(const orc_desc *d, const double *H, const int32_t *idx, int64_t k, double *w) {
    if (d->router_fn == ORC_ROUTER_SIGMOID) {
        double sum = 0.0;
        for (int64_t j = 0; j < k; ++j) sum += H[idx[j]];
        for (int64_t j = 0; j < k; ++j) w[j] = H[idx[j]] / (sum + 1e-15) * d->rsf;
    } else {
        orc_softmax_kept(H, idx, k, w);
    }
}

/* Router of one token: FP32 logits l (fp64 dot rounded to fp32), scores,
 * top-k of the selection scores (or the forced experts), weights. */
static void route(const orc_desc *d, const orc_tensors *w, const double *u, const int32_t *forced,
                  float *logits_out, int32_t *idx, double *wt, double *margin) {
    int64_t n = d->n, k = d->k;
    double *l = (double *)malloc(sizeof(double) * (size_t)n);
    float *lf = (float *)malloc(sizeof(float) * (size_t)n);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double *H = (double *)malloc(sizeof(double) * (size_t)n);
    matvec(w->router_w, d->rdt, n, d->d, 0, n, u, l);
    for (int64_t e = 0; e < n; ++e) {
        lf[e] = (float)l[e];
        if (logits_out) logits_out[e] = lf[e];
    }
    orc_router_scores(d, lf, w->bias, s, H);
    if (forced) {
        memcpy(idx, forced, sizeof(int32_t) * (size_t)k);
        if (margin) *margin = NAN;
    } else {
        orc_topk(s, n, k, idx, margin);
    }
    orc_router_weights(d, H, idx, k, wt);
    free(l);
    free(lf);
    free(s);
    free(H);
}

/* ------------------------------------------------------------------ */
/* Residual gate ([Gates] "Residual gates: derive the advertised       */
/* intuition carefully"; [FactSheet] residual design), coordinate-wise */
/* with w = g / tau: beta = sigmoid(w), alpha = sqrt(max(sigmoid(-w) * */
/* (1 + beta), floor)); out = alpha * r + beta * b.  The product is    */
/* evaluated as written, not rewritten as 1 - beta^2.                  */
/* ------------------------------------------------------------------ */
void orc_muse_gate_coeffs(double g, double tau, double floor_, double *alpha, double *beta) {
    double wv = g / tau;
    double b = 1.0 / (1.0 + exp(-wv));
    double sn = 1.0 / (1.0 + exp(wv));
    double a2 = sn * (1.0 + b);
    *beta = b;
    *alpha = sqrt(a2 > floor_ ? a2 : floor_);
}

/* Expert e applied to its input v (z for SwiGLU experts, u for ReLU
 * experts); o receives the expert output (length = L, or d without latent).
 * aout (may be NULL) receives the hidden activation a the second matrix
 * reads; a_given (may be NULL) is used as that activation instead of
 * computing it. */
static void expert(const orc_desc *d, const orc_tensors *w, int64_t e, const double *v, double *o, double *aout,
                   const double *a_given) {
    int64_t F = d->F;
    int64_t Kin = d->L ? d->L : d->d;   /* expert input width */
    int64_t Dout = Kin;                  /* expert output width */
    double *a = (double *)malloc(sizeof(double) * (size_t)F);
    if (a_given) {
        memcpy(a, a_given, sizeof(double) * (size_t)F);
    } else if (d->kind == ORC_SWIGLU) {
        double *g = (double *)malloc(sizeof(double) * (size_t)F);
        double *up = (double *)malloc(sizeof(double) * (size_t)F);
        int64_t rows1 = d->n * 2 * F;
        matvec(w->w1, d->wdt, rows1, Kin, e * 2 * F, F, v, g);
        matvec(w->w1, d->wdt, rows1, Kin, e * 2 * F + F, F, v, up);
        for (int64_t i = 0; i < F; ++i) {
            double silu = g[i] / (1.0 + exp(-g[i])); /* silu(t) = t * sigmoid(t) */
            a[i] = silu * up[i];
            if (d->mirror) a[i] = round_act(d->interm, a[i]);
        }
        quantize_activations(d, a, F);
        free(g);
        free(up);
    } else {
        matvec(w->w1, d->wdt, d->n * F, Kin, e * F, F, v, a);
        for (int64_t i = 0; i < F; ++i) {
            a[i] = a[i] > 0.0 ? a[i] : 0.0;
            if (d->mirror) a[i] = round_act(d->interm, a[i]);
        }
    }
    if (aout) memcpy(aout, a, sizeof(double) * (size_t)F);
    matvec(w->w2, d->wdt, d->n * Dout, F, e * Dout, Dout, a, o);
    free(a);
}

/* Per-expert output norm ([Gates], latent-experts section): the shared
 * normaliser applied to each expert output before its routing weight. */
static void expert_norm(const orc_desc *d, const orc_tensors *w, const double *o, int64_t D, double *nrm) {
    apply_norm(d->ex_norm, o, w->gamma_ex, D, d->eps_ex, d->act, nrm);
}

/*
 * Forward pass for tokens tok[0..ntok).  Outputs (each may be NULL):
 *   y     [ntok][d]  the branch output b that enters the residual gate:
 *                    P_up( sum_j w_j N(E_j(z)) ) ([Shazeer] y = sum_i
 *                    G(x)_i E_i(x); the up-projection is linear, so it is
 *                    applied once after the sum), then the FFN output norm
 *                    when out_norm is set ([Gates] "The complete layer has
 *                    two separately normalized residual updates")
 *   out   [ntok][d]  b, h + g * b (linear gate) or alpha * h + beta * b
 *                    (Muse gate), h = x
 *   ypre  [ntok][d]  P_up m, the branch output before the output norm
 *   logits[ntok][n]  fp32 router logits
 *   idx   [ntok][k]  selected experts, selection order
 *   wts   [ntok][k]  their gate weights
 *   margin[ntok]     k-th minus (k+1)-th selection score
 *   zout  [ntok][Dx] the expert-space input the experts read (the latent z
 *                    after the optional pre-norm and activation quantizer)
 * forced: [ntok][k] expert ids to use instead of the top-k (NULL: route).
 * forced_z: [ntok][Dx] expert-space inputs to use instead of computing them
 *        (NULL: compute), e.g. a device's quantized latent, the way forced
 *        evaluates a token on given experts.
 *   aout  [ntok][k][F] the hidden activation each selected expert's second
 *                    matrix reads (after the activation quantizer)
 * forced_a: [ntok][k][F] hidden activations to use instead of computing them
 *        (NULL: compute; not with dense).
 * dense: 1 evaluates every expert and sums G_e * N(E_e) over all n experts
 *        with the dense gate vector (zeros included): the brute-force form.
 */
int orc_forward(const orc_desc *d, const orc_tensors *w, const int64_t *tok, int64_t ntok,
                const int32_t *forced, int32_t dense, double *y, double *out, float *logits,
                int32_t *idx, double *wts, double *margin, double *ypre, double *zout,
                const double *forced_z, double *aout, const double *forced_a) {
    int64_t D = d->d, L = d->L, k = d->k, n = d->n;
    int64_t Dx = L ? L : D; /* width of the expert space */
    double *h = (double *)malloc(sizeof(double) * (size_t)D);
    double *u = (double *)malloc(sizeof(double) * (size_t)D);
    double *z = (double *)malloc(sizeof(double) * (size_t)Dx);
    double *o = (double *)malloc(sizeof(double) * (size_t)Dx);
    double *nr = (double *)malloc(sizeof(double) * (size_t)Dx);
    double *m = (double *)malloc(sizeof(double) * (size_t)Dx);
    double *yy = (double *)malloc(sizeof(double) * (size_t)D);
    double *bb = (double *)malloc(sizeof(double) * (size_t)D);
    double *zn = (double *)malloc(sizeof(double) * (size_t)Dx);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double *wt = (double *)malloc(sizeof(double) * (size_t)k);
    double *G = (double *)malloc(sizeof(double) * (size_t)n);
    for (int64_t q = 0; q < ntok; ++q) {
        int64_t t = tok ? tok[q] : q;
        branch_input(d, w, t, h, u);
        double mg;
        route(d, w, u, forced ? forced + q * k : NULL, logits ? logits + q * n : NULL, sel, wt, &mg);
        if (idx) memcpy(idx + q * k, sel, sizeof(int32_t) * (size_t)k);
        if (wts) memcpy(wts + q * k, wt, sizeof(double) * (size_t)k);
        if (margin) margin[q] = mg;
        if (!y && !out && !ypre && !zout && !aout) continue;
        /* expert-space input (or the given one) */
        if (forced_z) {
            memcpy(z, forced_z + q * Dx, sizeof(double) * (size_t)Dx);
        } else if (L) {
            matvec(w->down_w, d->wdt, L, D, 0, L, u, z);
            if (d->mirror) for (int64_t i = 0; i < L; ++i) z[i] = round_act(d->interm, z[i]);
            if (d->lat_norm != ORC_NORM_NONE) {
                /* z = C_pre(P_down u) ([Gates] latent-experts section) */
                apply_norm(d->lat_norm, z, w->gamma_lat, L, d->eps_lat, d->act, zn);
                memcpy(z, zn, sizeof(double) * (size_t)L);
                if (d->mirror) for (int64_t i = 0; i < L; ++i) z[i] = round_act(d->interm, z[i]);
            }
            quantize_activations(d, z, L);
        } else {
            memcpy(z, u, sizeof(double) * (size_t)D);
        }
        if (zout) memcpy(zout + q * Dx, z, sizeof(double) * (size_t)Dx);
        for (int64_t i = 0; i < Dx; ++i) m[i] = 0.0;
        if (dense) {
            for (int64_t e = 0; e < n; ++e) G[e] = 0.0;
            for (int64_t j = 0; j < k; ++j) G[sel[j]] = wt[j];
            for (int64_t e = 0; e < n; ++e) {
                expert(d, w, e, z, o, NULL, NULL);
                expert_norm(d, w, o, Dx, nr);
                for (int64_t i = 0; i < Dx; ++i) m[i] += G[e] * nr[i];
            }
        } else {
            for (int64_t j = 0; j < k; ++j) {
                expert(d, w, sel[j], z, o, aout ? aout + (q * k + j) * d->F : NULL,
                       forced_a ? forced_a + (q * k + j) * d->F : NULL);
                expert_norm(d, w, o, Dx, nr);
                for (int64_t i = 0; i < Dx; ++i) m[i] += wt[j] * nr[i];
            }
        }
        if (d->mirror) for (int64_t i = 0; i < Dx; ++i) m[i] = round_act(d->interm, m[i]);
        if (L) matvec(w->up_w, d->wdt, D, L, 0, D, m, yy);
        else memcpy(yy, m, sizeof(double) * (size_t)D);
        if (ypre) memcpy(ypre + q * D, yy, sizeof(double) * (size_t)D);
        apply_norm(d->out_norm, yy, w->gamma_out, D, d->eps_out, d->act, bb);
        if (y) memcpy(y + q * D, bb, sizeof(double) * (size_t)D);
        if (out) {
            for (int64_t i = 0; i < D; ++i) {
                double r;
                if (d->res_gate == ORC_RES_LINEAR) {
                    r = h[i] + (double)w->gate[i] * bb[i];
                } else if (d->res_gate == ORC_RES_MUSE) {
                    double al, be;
                    orc_muse_gate_coeffs((double)w->gate[i], d->tau, d->floor_, &al, &be);
                    r = al * h[i] + be * bb[i];
                } else {
                    r = bb[i];
                }
                out[q * D + i] = r;
            }
        }
    }
    free(h); free(u); free(z); free(o); free(nr); free(m); free(yy); free(bb); free(zn); free(sel); free(wt);
    free(G);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Permutation: the (token, slot) pairs grouped by expert, ascending   */
/* expert then ascending token (a token never picks an expert twice,   */
/* so the order is unique).                                            */
/* ------------------------------------------------------------------ */
int orc_permute(const int32_t *idx, int64_t T, int64_t k, int64_t n, int32_t *counts, int32_t *offsets,
                int32_t *perm_tok, int32_t *perm_slot, int32_t *pos) {
    for (int64_t e = 0; e < n; ++e) counts[e] = 0;
    for (int64_t i = 0; i < T * k; ++i) {
        if (idx[i] < 0 || idx[i] >= n) return -1;
        counts[idx[i]]++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < n; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t p = 0;
    for (int64_t e = 0; e < n; ++e)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < k; ++j)
                if (idx[t * k + j] == e) {
                    perm_tok[p] = (int32_t)t;
                    perm_slot[p] = (int32_t)j;
                    pos[t * k + j] = (int32_t)p;
                    ++p;
                }
    return 0;
}

/* Decode a whole stored weight matrix to doubles (for pins and small cases). */
void orc_decode_matrix(const void *base, int32_t dt, int64_t rows, int64_t K, double *out) {
    for (int64_t r = 0; r < rows; ++r) load_row(base, dt, rows, K, r, out + r * K);
}

double orc_round_bf16(double v) { return round_to_bf16(v); }
double orc_round_f16(double v) { return round_to_f16(v); }

/* The branch input u (x, or its input norm in the input dtype) of tokens
 * tok[0..ntok), as the forward pass computes it: out [ntok][d]. */
void orc_branch_input(const orc_desc *d, const orc_tensors *w, const int64_t *tok, int64_t ntok, double *out) {
    double *h = (double *)malloc(sizeof(double) * (size_t)d->d);
    for (int64_t q = 0; q < ntok; ++q) branch_input(d, w, tok[q], h, out + q * d->d);
    free(h);
}

/* Threads of the oracle's parallel row loops (the OpenMP team size; 1 without OpenMP). */
int orc_threads(void) {
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
