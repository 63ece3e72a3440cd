/*
 * NVFP4 activation-quantization oracle (plain C, single-threaded).
 * TEST INFRASTRUCTURE ONLY -- see nvfp4_oracle.h for scope, sources and the
 * readings taken where the pages are silent.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (x86-64 SSE, so
 * every float operation below is one correctly rounded binary32 operation).
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Bit views                                                                 */
/* ------------------------------------------------------------------------ */
static float f32_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ------------------------------------------------------------------------ */
/* BF16 <-> binary32                                                         */
/* ------------------------------------------------------------------------ */
float ora_bf16_to_f32(uint16_t h) { return f32_of((uint32_t)h << 16); }

/* Value of a bf16 magnitude pattern (0..0x7F80) as a double; the pattern
 * 0x7F80 is treated as 2^128, the next value beyond the largest finite bf16
 * with an unbounded exponent, so that rounding into it means overflow to inf
 * exactly as IEEE 754 round-to-nearest specifies. */
static double bf16_mag_value(uint16_t p) {
    if (p == 0x7F80) return ldexp(1.0, 128);
    return (double)ora_bf16_to_f32(p);
}

/* Nearest bf16 to f, ties to the even pattern.  The two candidates are the
 * magnitude truncated to 16 bits and its successor; every distance is exact in
 * double because f and both candidates share a binade up to a factor 2. */
uint16_t ora_f32_to_bf16(float f) {
    uint32_t u = bits_of(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040); /* NaN: quiet, sign kept */
    if (mag == 0x7F800000u) return (uint16_t)(sign | 0x7F80);
    uint16_t lo = (uint16_t)(mag >> 16);
    uint16_t hi = (uint16_t)(lo + 1);
    double a = fabs((double)f);
    double dlo = a - bf16_mag_value(lo);
    double dhi = bf16_mag_value(hi) - a;
    uint16_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = (lo & 1) ? hi : lo;
    return (uint16_t)(sign | pick);
}

/* ------------------------------------------------------------------------ */
/* E4M3FN (OCP FP8): 1 sign, 4 exponent (bias 7), 3 mantissa bits.           */
/* Finite magnitudes: subnormals m * 2^-9, normals (1 + m/8) * 2^(e-7),      */
/* largest 448 (0x7E); 0x7F is NaN.                                          */
/* ------------------------------------------------------------------------ */
double ora_e4m3_value(uint8_t code) {
    int e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if ((code & 0x7F) == 0x7F) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return (code & 0x80) ? -v : v;
}

/* Unsigned block-scale encoder: nearest of the 127 finite non-negative E4M3
 * values by exhaustive search, ties to the even code; t >= 448 (including
 * +inf) saturates to 448; NaN -> 0x7F; t <= 0 -> 0. */
uint8_t ora_e4m3_encode(float t) {
    if (isnan(t)) return 0x7F;
    if (t <= 0.0f) return 0x00;
    if (t >= 448.0f) return 0x7E;
    double a = (double)t;
    int best = 0;
    double bestd = a; /* distance to code 0 (value 0) */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - ora_e4m3_value((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------------------------------ */
/* E2M1 (FP4): 1 sign, 2 exponent, 1 mantissa bit.                           */
/* Codes 0..7 = magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 = sign.        */
/* ------------------------------------------------------------------------ */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double ora_e2m1_value(uint8_t code) {
    double v = kE2M1[code & 7];
    return (code & 8) ? -v : v;
}

/* Nearest magnitude, ties to the even code, |v| >= 6 -> 6, the sign bit of v
 * is kept (so -0 and small negatives give 0x8); NaN -> 0x0. */
uint8_t ora_e2m1_encode(float v) {
    if (isnan(v)) return 0x0;
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs((double)v);
    if (a >= 6.0) return (uint8_t)(sign | 7);
    int best = 0;
    double bestd = a;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - kE2M1[c]);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------------ */
/* Element steps                                                             */
/* ------------------------------------------------------------------------ */

/* AdaLN modulation with BF16 rounding after each of the three operations,
 * in the order (x * (scale + 1)) + shift ("NVFP4 Modulation Producer Fusion",
 * Exactness Contract). */
uint16_t ora_modulate(uint16_t x, uint16_t scale, uint16_t shift) {
    float s1 = ora_bf16_to_f32(scale) + 1.0f;
    float s1b = ora_bf16_to_f32(ora_f32_to_bf16(s1));
    float p = ora_bf16_to_f32(x) * s1b;
    float pb = ora_bf16_to_f32(ora_f32_to_bf16(p));
    float y = pb + ora_bf16_to_f32(shift);
    return ora_f32_to_bf16(y);
}

/* Correctly rounded binary32 exp(-g): the binary64 exp is within one binary64
 * ulp, and for every bf16 g the exact value lies far enough from a binary32
 * rounding midpoint that rounding the binary64 result gives the correctly
 * rounded binary32 value (checked against multiprecision in the tests). */
float ora_exp_neg(uint16_t g) {
    double gd = (double)ora_bf16_to_f32(g);
    return (float)exp(-gd);
}

/* silu(g) = g / (1 + exp(-g)) in binary32, rounded to bf16 ("FC2 NVFP4 Library
 * Scheduling", Exact Operation / Current Baseline: exact BF16 SwiGLU). */
uint16_t ora_silu_bf16(uint16_t g) {
    float gf = ora_bf16_to_f32(g);
    float e = ora_exp_neg(g);
    float den = 1.0f + e;
    float sl = gf / den;
    return ora_f32_to_bf16(sl);
}

uint16_t ora_swiglu(uint16_t g, uint16_t u) {
    float sb = ora_bf16_to_f32(ora_silu_bf16(g));
    float h = sb * ora_bf16_to_f32(u);
    return ora_f32_to_bf16(h);
}

/* One FP32 tensor scale from the global absolute maximum ("NVFP4 Streaming
 * Design", Numerical Constraint): amax / (6 * 448), or 1 when amax is 0. */
float ora_tensor_scale(float amax) {
    if (amax == 0.0f) return 1.0f;
    return amax / 2688.0f;
}

/* The E4M3 scale of a 16-value block: E4M3(RN(RN(a16 / 6) / s_g)). */
uint8_t ora_block_scale(float a16, float s_g) {
    float t6 = a16 / 6.0f;
    float t = t6 / s_g;
    return ora_e4m3_encode(t);
}

/* E2M1 value quantized with both scales: E2M1(RN(y / RN(sf * s_g))). */
uint8_t ora_element_code(uint16_t y, uint8_t sf, float s_g) {
    if (sf == 0) return 0;
    float sff = (float)ora_e4m3_value(sf);
    float d = sff * s_g;
    float q = ora_bf16_to_f32(y) / d;
    return ora_e2m1_encode(q);
}

/* ------------------------------------------------------------------------ */
/* Tensor passes                                                             */
/* ------------------------------------------------------------------------ */
static int32_t segment_of(int64_t r, int32_t nseg, const int64_t* row_start) {
    int32_t s = 0;
    while (s + 1 < nseg && r >= row_start[s + 1]) ++s;
    return s;
}

/* |y| compared as bf16 magnitude bit patterns: for finite values this is the
 * ordinary absolute-value order, and it ranks NaN above Inf above finite. */
static uint16_t mag16(uint16_t y) { return (uint16_t)(y & 0x7FFF); }

/* Quantize one 16-value block of bf16 y into 8 packed bytes and its scale. */
static void pack_block(const uint16_t y[16], float s_g, uint8_t* q8, uint8_t* sf_out) {
    uint16_t m = 0;
    for (int i = 0; i < 16; ++i)
        if (mag16(y[i]) > m) m = mag16(y[i]);
    float a16 = ora_bf16_to_f32(m);
    uint8_t sf = ora_block_scale(a16, s_g);
    *sf_out = sf;
    for (int j = 0; j < 8; ++j) {
        uint8_t lo = ora_element_code(y[2 * j], sf, s_g);
        uint8_t hi = ora_element_code(y[2 * j + 1], sf, s_g);
        q8[j] = (uint8_t)(lo | (hi << 4));
    }
}

float ora_modulate_amax(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                        int32_t nseg, const int64_t* row_start,
                        const uint16_t* shift, const uint16_t* scale, int64_t ld_seg) {
    return ora_modulate_amax_rows(x, D, ldx, nseg, row_start, shift, scale, ld_seg, 0, M);
}

float ora_modulate_amax_rows(const uint16_t* x, int64_t D, int64_t ldx,
                             int32_t nseg, const int64_t* row_start,
                             const uint16_t* shift, const uint16_t* scale, int64_t ld_seg,
                             int64_t r0, int64_t r1) {
    uint16_t m = 0;
    for (int64_t r = r0; r < r1; ++r) {
        int32_t s = segment_of(r, nseg, row_start);
        for (int64_t c = 0; c < D; ++c) {
            uint16_t y = ora_modulate(x[r * ldx + c], scale[s * ld_seg + c], shift[s * ld_seg + c]);
            if (mag16(y) > m) m = mag16(y);
        }
    }
    return ora_bf16_to_f32(m);
}

void ora_modulate_pack_rows(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                            int32_t nseg, const int64_t* row_start,
                            const uint16_t* shift, const uint16_t* scale, int64_t ld_seg,
                            float s_g, int64_t r0, int64_t r1,
                            uint8_t* qdata, uint8_t* sfa) {
    uint16_t y[16];
    for (int64_t r = r0; r < r1; ++r) {
        uint8_t* qrow = qdata + (r - r0) * (D / 2);
        uint8_t* srow = sfa + (r - r0) * (D / 16);
        if (r >= M) {
            memset(qrow, 0, (size_t)(D / 2));
            memset(srow, 0, (size_t)(D / 16));
            continue;
        }
        int32_t s = segment_of(r, nseg, row_start);
        for (int64_t b = 0; b < D / 16; ++b) {
            for (int i = 0; i < 16; ++i) {
                int64_t c = b * 16 + i;
                y[i] = ora_modulate(x[r * ldx + c], scale[s * ld_seg + c], shift[s * ld_seg + c]);
            }
            pack_block(y, s_g, qrow + b * 8, srow + b);
        }
    }
}

float ora_swiglu_amax(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F, int64_t ld) {
    return ora_swiglu_amax_rows(gate, up, F, ld, 0, M);
}

float ora_swiglu_amax_rows(const uint16_t* gate, const uint16_t* up, int64_t F, int64_t ld, int64_t r0, int64_t r1) {
    uint16_t m = 0;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = 0; c < F; ++c) {
            uint16_t h = ora_swiglu(gate[r * ld + c], up[r * ld + c]);
            if (mag16(h) > m) m = mag16(h);
        }
    return ora_bf16_to_f32(m);
}

void ora_swiglu_pack_rows(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F, int64_t ld,
                          float s_g, int64_t r0, int64_t r1, uint8_t* qdata, uint8_t* sfa) {
    uint16_t h[16];
    for (int64_t r = r0; r < r1; ++r) {
        uint8_t* qrow = qdata + (r - r0) * (F / 2);
        uint8_t* srow = sfa + (r - r0) * (F / 16);
        if (r >= M) {
            memset(qrow, 0, (size_t)(F / 2));
            memset(srow, 0, (size_t)(F / 16));
            continue;
        }
        for (int64_t b = 0; b < F / 16; ++b) {
            for (int i = 0; i < 16; ++i) {
                int64_t c = b * 16 + i;
                h[i] = ora_swiglu(gate[r * ld + c], up[r * ld + c]);
            }
            pack_block(h, s_g, qrow + b * 8, srow + b);
        }
    }
}

float ora_bf16_amax(const uint16_t* y, int64_t M, int64_t D, int64_t ldy) {
    uint16_t m = 0;
    for (int64_t r = 0; r < M; ++r)
        for (int64_t c = 0; c < D; ++c)
            if (mag16(y[r * ldy + c]) > m) m = mag16(y[r * ldy + c]);
    return ora_bf16_to_f32(m);
}

void ora_bf16_pack_rows(const uint16_t* y, int64_t M, int64_t D, int64_t ldy, float s_g,
                        int64_t r0, int64_t r1, uint8_t* qdata, uint8_t* sfa) {
    for (int64_t r = r0; r < r1; ++r) {
        uint8_t* qrow = qdata + (r - r0) * (D / 2);
        uint8_t* srow = sfa + (r - r0) * (D / 16);
        if (r >= M) {
            memset(qrow, 0, (size_t)(D / 2));
            memset(srow, 0, (size_t)(D / 16));
            continue;
        }
        for (int64_t b = 0; b < D / 16; ++b) pack_block(y + r * ldy + b * 16, s_g, qrow + b * 8, srow + b);
    }
}

/* ------------------------------------------------------------------------ */
/* Elementwise batches                                                       */
/* ------------------------------------------------------------------------ */
void ora_modulate_batch(const uint16_t* x, const uint16_t* scale, const uint16_t* shift, int64_t n, uint16_t* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = ora_modulate(x[i], scale[i], shift[i]);
}

void ora_swiglu_batch(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = ora_swiglu(g[i], u[i]);
}

/* a16 given as bf16 bits; its magnitude is used. */
void ora_block_scale_batch(const uint16_t* a16, int64_t n, float s_g, uint8_t* sf) {
    for (int64_t i = 0; i < n; ++i) sf[i] = ora_block_scale(ora_bf16_to_f32(mag16(a16[i])), s_g);
}

void ora_element_code_batch(const uint16_t* y, const uint8_t* sf, int64_t n, float s_g, uint8_t* code) {
    for (int64_t i = 0; i < n; ++i) code[i] = ora_element_code(y[i], sf[i], s_g);
}

void ora_e2m1_encode_batch(const float* v, int64_t n, uint8_t* code) {
    for (int64_t i = 0; i < n; ++i) code[i] = ora_e2m1_encode(v[i]);
}

void ora_e4m3_encode_batch(const float* t, int64_t n, uint8_t* code) {
    for (int64_t i = 0; i < n; ++i) code[i] = ora_e4m3_encode(t[i]);
}

/* ------------------------------------------------------------------------ */
/* Exact residual epilogue ("NVFP4 Streaming Design", P4): the GEMM result  */
/* rounded to BF16, times the gate, plus the residual, rounded again         */
/* ------------------------------------------------------------------------ */
uint16_t ora_gate_residual(uint16_t o, uint16_t gate, uint16_t residual) {
    float g = ora_bf16_to_f32(gate) * ora_bf16_to_f32(o);
    float gb = ora_bf16_to_f32(ora_f32_to_bf16(g));
    float r = ora_bf16_to_f32(residual) + gb;
    return ora_f32_to_bf16(r);
}

void ora_gate_residual_rows(const uint16_t* o, int64_t M, int64_t N, int64_t ldo,
                            int32_t nseg, const int64_t* row_start, const uint16_t* gate, int64_t ld_gate,
                            const uint16_t* residual, int64_t ldr, uint16_t* out, int64_t ld_out) {
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* grow = gate + (int64_t)segment_of(m, nseg, row_start) * ld_gate;
        for (int64_t n = 0; n < N; ++n)
            out[m * ld_out + n] = ora_gate_residual(o[m * ldo + n], grow[n], residual[m * ldr + n]);
    }
}

/* ------------------------------------------------------------------------ */
/* GEMM reference                                                            */
/* ------------------------------------------------------------------------ */
static double decoded(const uint8_t* q, const uint8_t* sf, int64_t row, int64_t k, int64_t K) {
    uint8_t byte = q[row * (K / 2) + k / 2];
    uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
    return ora_e2m1_value(code) * ora_e4m3_value(sf[row * (K / 16) + k / 16]);
}

#include <stdlib.h>

void ora_gemm_rows(const uint8_t* qa, const uint8_t* sfa, float a_scale,
                   const uint8_t* qw, const uint8_t* sfw, float w_scale,
                   int64_t N, int64_t K, const int64_t* rows, int64_t nrows, double* out) {
    float alpha = a_scale * w_scale;
    double* arow = (double*)malloc(sizeof(double) * (size_t)(nrows * K));
    double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t k = 0; k < K; ++k) arow[i * K + k] = decoded(qa, sfa, rows[i], k, K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) wrow[k] = decoded(qw, sfw, n, k, K);
        for (int64_t i = 0; i < nrows; ++i) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += arow[i * K + k] * wrow[k];
            out[i * N + n] = (double)alpha * s;
        }
    }
    free(wrow);
    free(arow);
}

void ora_gemm_bf16_rows(const uint8_t* qa, const uint8_t* sfa, float a_scale,
                        const uint8_t* qw, const uint8_t* sfw, float w_scale,
                        int64_t N, int64_t K, const int64_t* rows, int64_t nrows, uint16_t* out) {
    /* the binary64 sums S (unit scales), then bf16(RN32(alpha * RN32(S))) */
    double* sums = (double*)malloc(sizeof(double) * (size_t)(nrows * N));
    ora_gemm_rows(qa, sfa, 1.0f, qw, sfw, 1.0f, N, K, rows, nrows, sums);
    float alpha = a_scale * w_scale;
    for (int64_t i = 0; i < nrows * N; ++i) {
        float sf = (float)sums[i];
        float o = alpha * sf;
        out[i] = ora_f32_to_bf16(o);
    }
    free(sums);
}
