/*
 * NVFP4 activation-quantization oracle: plain, slow, single-threaded C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; neither side
 * includes or links the other.
 *
 * Every floating-point step is IEEE binary32 with round-to-nearest-even,
 * written one operation per statement and compiled without FMA contraction or
 * fast-math, so each step is exactly the correctly rounded operation the
 * definition names.  The GEMM reference accumulates in binary64.
 *
 * Sources (page title, section):
 *  - "NVFP4 Modulation Producer Fusion", Exactness Contract: per-segment
 *    shift/scale selection, the (x*(scale+1))+shift order with BF16 rounding.
 *  - "NVFP4 Streaming Design", Numerical Constraint: the tensor's exact BF16
 *    maximum magnitude gives a single FP32 tensor scale; each 16 values get
 *    an E4M3 scale; E2M1 codes come from both scales; no tile can
 *    be packed before the global reduction completes.
 *  - "FC2 NVFP4 Library Scheduling", Exact Operation: packed activation rows
 *    [M,K] against packed weight rows [N,K], giving BF16 [M,N], FP32 compute,
 *    alpha = activation tensor scale * weight tensor scale, 37,810 rows padded
 *    to 37,824; exact BF16 SwiGLU feeding the FC2 producer.
 *
 * Where the pages leave a step open this oracle takes one fixed reading:
 * s_g = amax/2688 (1 when amax = 0); sf = E4M3(RN(RN(a16/6)/s_g)) with
 * round-to-nearest-even and saturation at 448; q = E2M1(RN(y/RN(sf*s_g)))
 * with ties to the even code, saturation at 6 and code 0 when sf = 0;
 * low nibble = even column; plain row-major scales; padded rows are zero;
 * silu(g) = g/(1+exp(-g)) with a correctly rounded binary32 exp.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar conversions ------------------------------------------------ */
float    ora_bf16_to_f32(uint16_t h);
uint16_t ora_f32_to_bf16(float f);          /* nearest, ties to even; NaN -> quiet NaN, sign kept */
double   ora_e4m3_value(uint8_t code);      /* E4M3FN: bias 7, max 448, 0x7F/0xFF = NaN */
uint8_t  ora_e4m3_encode(float t);          /* t >= 0: nearest finite value, ties to even code, >= 448 -> 0x7E */
double   ora_e2m1_value(uint8_t code);      /* {0,.5,1,1.5,2,3,4,6}, bit 3 = sign */
uint8_t  ora_e2m1_encode(float v);          /* nearest, ties to even code, |v| >= 6 -> 6, NaN -> 0 */

/* ---- element steps ----------------------------------------------------- */
uint16_t ora_modulate(uint16_t x, uint16_t scale, uint16_t shift);  /* bf16((bf16(x*bf16(scale+1)))+shift) */
float    ora_exp_neg(uint16_t g);           /* binary32 exp(-g), correctly rounded */
uint16_t ora_silu_bf16(uint16_t g);         /* bf16(g / (1 + exp(-g))) */
uint16_t ora_swiglu(uint16_t g, uint16_t u);/* bf16(silu_bf16(g) * u) */
float    ora_tensor_scale(float amax);      /* amax == 0 ? 1 : amax / 2688 */
uint8_t  ora_block_scale(float a16, float s_g);                 /* E4M3(RN(RN(a16/6)/s_g)) */
uint8_t  ora_element_code(uint16_t y, uint8_t sf, float s_g);   /* E2M1(RN(y/RN(sf*s_g))), 0 if sf == 0 */

/* ---- tensor passes ----------------------------------------------------- *
 * Segments: nseg contiguous row ranges [row_start[s], row_start[s+1]) with
 * row_start[0] = 0 and row_start[nseg] = M; shift/scale are [nseg, D] bf16
 * with row stride ld_seg.  x is [M, D] bf16 with row stride ldx.            */
float ora_modulate_amax(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                        int32_t nseg, const int64_t* row_start,
                        const uint16_t* shift, const uint16_t* scale, int64_t ld_seg);
/* max |y| over rows [r0, r1) only (the full maximum is the max over row ranges). */
float ora_modulate_amax_rows(const uint16_t* x, int64_t D, int64_t ldx,
                             int32_t nseg, const int64_t* row_start,
                             const uint16_t* shift, const uint16_t* scale, int64_t ld_seg,
                             int64_t r0, int64_t r1);
/* Writes rows [r0, r1) of qdata [*, D/2] and sfa [*, D/16]; rows >= M are zero-filled. */
void ora_modulate_pack_rows(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                            int32_t nseg, const int64_t* row_start,
                            const uint16_t* shift, const uint16_t* scale, int64_t ld_seg,
                            float s_g, int64_t r0, int64_t r1,
                            uint8_t* qdata, uint8_t* sfa);
/* gate/up: [M, F] bf16 views with row stride ld (for one [M, 2F] tensor: up = gate + F, ld = 2F). */
float ora_swiglu_amax(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F, int64_t ld);
float ora_swiglu_amax_rows(const uint16_t* gate, const uint16_t* up, int64_t F, int64_t ld, int64_t r0, int64_t r1);
void  ora_swiglu_pack_rows(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F, int64_t ld,
                           float s_g, int64_t r0, int64_t r1, uint8_t* qdata, uint8_t* sfa);
/* Quantize an already-formed bf16 tensor y [M, D] (row stride ldy). */
float ora_bf16_amax(const uint16_t* y, int64_t M, int64_t D, int64_t ldy);
void  ora_bf16_pack_rows(const uint16_t* y, int64_t M, int64_t D, int64_t ldy, float s_g,
                         int64_t r0, int64_t r1, uint8_t* qdata, uint8_t* sfa);

/* ---- elementwise batches (plain loops over the scalar steps) --------- */
void ora_modulate_batch(const uint16_t* x, const uint16_t* scale, const uint16_t* shift, int64_t n, uint16_t* y);
void ora_swiglu_batch(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* h);
void ora_block_scale_batch(const uint16_t* a16, int64_t n, float s_g, uint8_t* sf);
void ora_element_code_batch(const uint16_t* y, const uint8_t* sf, int64_t n, float s_g, uint8_t* code);
void ora_e2m1_encode_batch(const float* v, int64_t n, uint8_t* code);
void ora_e4m3_encode_batch(const float* t, int64_t n, uint8_t* code);

/* ---- exact residual epilogue ("NVFP4 Streaming Design", P4) -------------- *
 * The GEMM's BF16 output o is scaled by the gate and added to the residual,
 * each step one binary32 operation rounded to BF16:
 *   out = bf16(residual + bf16(gate * o))                                   */
uint16_t ora_gate_residual(uint16_t o, uint16_t gate, uint16_t residual);
/* The same over o [M, N] (row stride ldo): gate is [nseg, N] bf16 (row stride
 * ld_gate), row m using the gate row of its segment; residual [M, N] (row
 * stride ldr); writes out [M, N] (row stride ld_out).                       */
void ora_gate_residual_rows(const uint16_t* o, int64_t M, int64_t N, int64_t ldo,
                            int32_t nseg, const int64_t* row_start, const uint16_t* gate, int64_t ld_gate,
                            const uint16_t* residual, int64_t ldr, uint16_t* out, int64_t ld_out);

/* ---- GEMM reference ----------------------------------------------------- *
 * out[i][n] = (double)RN32(a_scale*w_scale) * sum_k A[rows[i]][k] * W[n][k]
 * with A = e2m1(qa)*e4m3(sfa), W = e2m1(qw)*e4m3(sfw), all in binary64.    */
void ora_gemm_rows(const uint8_t* qa, const uint8_t* sfa, float a_scale,
                   const uint8_t* qw, const uint8_t* sfw, float w_scale,
                   int64_t N, int64_t K, const int64_t* rows, int64_t nrows, double* out);
/* The BF16 output bf16(RN32(RN32(a_scale*w_scale) * RN32(S))) with S the
 * binary64 sum above rounded once to binary32: the GEMM's BF16 output
 * whenever the binary32 accumulation of the sum is exact (for example when
 * every output is a single product, as with an identity weight).            */
void ora_gemm_bf16_rows(const uint8_t* qa, const uint8_t* sfa, float a_scale,
                        const uint8_t* qw, const uint8_t* sfw, float w_scale,
                        int64_t N, int64_t K, const int64_t* rows, int64_t nrows, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
