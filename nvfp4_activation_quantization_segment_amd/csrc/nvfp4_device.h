// Device-side numerics of the NVFP4 producer for gfx950 (CDNA4).
//
// Every function here is a correctly rounded binary32 computation of one step
// of the quantizer (no FMA contraction, no flush-to-zero), built from gfx950
// instructions whose rounding is checked over the step's whole input domain by
// the single-step entry points.
//
// Sources (page title, section):
//   "NVFP4 Modulation Producer Fusion", Exactness Contract -- the BF16
//     modulation (x * (scale + 1)) + shift with BF16 rounding.
//   "NVFP4 Streaming Design", Numerical Constraint -- global amax, FP32 tensor
//     scale, one E4M3 scale per 16 values, E2M1 values with both scales.
//   "FC2 NVFP4 Library Scheduling", Current Baseline -- exact BF16 SwiGLU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Streaming stores.  Outputs that no later step of the same kernel reads are
// written non-temporally where a wave's store covers whole cache lines: plain
// stores leave dirty lines in the memory-side cache, and the next kernel's
// reads then share the bandwidth with their write-back (a 406 MB read after a
// 1 GB write took 2.3x as long).  Stores that cover only parts of lines (the
// bytes of a scale row) stay plain, so that the L2 merges them first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_nt(uint2* p, uint2 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------------------
// BF16 <-> binary32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two binary32 -> two bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32);
// a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// RN(a) to bf16, returned as the binary32 value it equals: v_cvt_pk_bf16_f32
// with a zero low half puts bf16(a) in the high half, which is that binary32
// bit pattern (one instruction instead of a convert and an unpack).
__device__ __forceinline__ float round_bf16(float a) { return __uint_as_float(pack_bf16x2(0.0f, a)); }

// ---------------------------------------------------------------------------
// Modulation: y = bf16(bf16(x * s1) + shift) with s1 = bf16(scale + 1)
// already formed.  Operates on two packed bf16 values.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float mod_scale1(uint16_t scale_bits) {
    float s = __uint_as_float((uint32_t)scale_bits << 16) + 1.0f;
    return bf16_lo(pack_bf16x2(s, s));
}

__device__ __forceinline__ uint32_t modulate2(uint32_t x2, float s1a, float s1b, float sha, float shb) {
    uint32_t p = pack_bf16x2(bf16_lo(x2) * s1a, bf16_hi(x2) * s1b);
    return pack_bf16x2(bf16_lo(p) + sha, bf16_hi(p) + shb);
}

// ---------------------------------------------------------------------------
// SwiGLU: h = bf16(bf16(silu(g)) * u), silu(g) = g / (1 + exp(-g)) with a
// correctly rounded binary32 exp, every step rounded to binary32, the quotient
// rounded to bf16.
//
// Exact path: the binary64 exp rounded to binary32 is the correctly rounded
// value for every bf16 g (the exact value is never within the binary64 error
// of a binary32 rounding midpoint); the rest follows the definition.
//
// Fast path (binary32 only): exp(-g) = 2^(a + b) with -g*log2(e) split so that
// a = -g * L2E_HI is exact (g has 8 significant bits, L2E_HI 15) and b is the
// small remainder; 2^(a - rint(a) + b) by v_exp_f32, scaled by 2^rint(a).
// The quotient uses v_rcp_f32 and one fma correction.  The result is within a
// few binary32 ulps of the exact chain, so it rounds to the same bf16 unless
// it lies within 16 ulps of a bf16 rounding midpoint; those values (and an
// overflowing exp) take the exact path.  Because g is bf16, the 65,536 inputs
// are checked exhaustively against the oracle.  The producer kernels evaluate
// this once per bf16 bit pattern into a lookup table at the start of a call.
// ---------------------------------------------------------------------------
constexpr float kL2eHi = 0x1.715400p+0f;   // log2(e) to 15 significant bits
constexpr float kL2eLo = 0x1.d94ae0p-18f;  // log2(e) - kL2eHi, rounded

__device__ __forceinline__ float silu_exact(float g) {
    float e = (float)exp(-(double)g);
    float den = 1.0f + e;
    return g / den;  // correctly rounded division
}

__device__ __forceinline__ float silu_bf16_value(float g) {
    float a = -g * kL2eHi;
    const float b = -g * kL2eLo;
    a = __builtin_fminf(__builtin_fmaxf(a, -160.0f), 130.0f);
    const float n = __builtin_rintf(a);
    const float f = (a - n) + b;
    const float e = __builtin_ldexpf(__builtin_amdgcn_exp2f(f), (int)n);
    const float den = 1.0f + e;
    const float r = __builtin_amdgcn_rcpf(den);
    const float q0 = g * r;
    const float e1 = __builtin_fmaf(q0, den, -g);  // residual form keeps the sign of g = -0
    float sl = __builtin_fmaf(-e1, r, q0);
    const uint32_t lo = __float_as_uint(sl) & 0xFFFFu;
    if ((lo - 0x7FF0u) <= 0x20u || !(den < 1e38f)) sl = silu_exact(g);
    return bf16_lo(pack_bf16x2(sl, sl));
}

// ---------------------------------------------------------------------------
// E4M3FN (bias 7, max 448, 0x7F = NaN)
// ---------------------------------------------------------------------------
// Non-negative t -> nearest E4M3 code, ties to even; t >= 448 -> 0x7E;
// NaN -> 0x7F.  On gfx950 v_cvt_pk_fp8_f32 converts to OCP E4M3FN with
// round-to-nearest-even (checked against the oracle on structured covers of
// every rounding case below 464); saturation and NaN are made explicit.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
    const float tc = t < 448.0f ? t : 448.0f;
    uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(tc, 0.0f, 0, false) & 0xFFu;
    return (t != t) ? 0x7Fu : code;
}

// E4M3 code -> its binary32 value (exact; v_cvt_f32_fp8 decodes OCP E4M3FN).
__device__ __forceinline__ float e4m3_value(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// ---------------------------------------------------------------------------
// Division by a block constant.
// For a correctly rounded reciprocal r = RN(1/d), the Markstein sequence
//   q0 = RN(y*r); e = RN(q0*d - y) (exact, one fma); q = RN(q0 - e*r)
// returns RN(y/d) whenever no intermediate overflows or underflows
// (P. Markstein, IBM J. Res. Dev. 34(1), 1990).  The residual is formed as
// q0*d - y rather than y - q0*d so that y = -0 yields -0 (an exact zero
// residual then enters as -0 and cannot flip the sign of q0).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float div_markstein(float y, float d, float r) {
    float q0 = y * r;
    float e = __builtin_fmaf(q0, d, -y);
    return __builtin_fmaf(-e, r, q0);
}

// RN(1/6) in binary32.
constexpr float kRcp6 = 0x1.555556p-3f;

// Block scale from the block maximum: E4M3(RN(RN(a16/6)/s_g)).  rg = RN(1/s_g).
// Valid for finite a16 >= 0 and s_g in the kernel's fast range.  Inside a
// tensor t <= 448 (up to rounding), but for an a16 far above 2688*s_g the
// first product may overflow; any t >= 1024 saturates to 448 anyway, so the
// uncorrected product is used there.
__device__ __forceinline__ uint32_t block_scale_fast(float a16, float s_g, float rg) {
    const float u = div_markstein(a16, 6.0f, kRcp6);
    const float q0 = u * rg;
    const float e = __builtin_fmaf(q0, s_g, -u);
    const float t = (q0 >= 1024.0f) ? q0 : __builtin_fmaf(-e, rg, q0);
    return e4m3_encode(t);
}

// The same inside a launch that took s_g from the maximum of the very values
// whose blocks it scales (a16 <= amax, s_g = RN(amax/2688) in the fast range):
// RN(a16/6) <= RN(amax/6), and its quotient by s_g is at most 448 (1 + 2^-22),
// so t < 464 always, the first product cannot overflow, and the clamp and
// NaN test of e4m3_encode never change the code.
__device__ __forceinline__ uint32_t block_scale_bounded(float a16, float s_g, float rg) {
    const float t = div_markstein(div_markstein(a16, 6.0f, kRcp6), s_g, rg);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false) & 0xFFu;
}

// Reference-form block scale with two correctly rounded divisions (any input).
__device__ __forceinline__ uint32_t block_scale_slow(float a16, float s_g) {
    float u = a16 / 6.0f;
    float t = u / s_g;
    return e4m3_encode(t);
}

// The fast path holds for 2^-80 <= s_g <= 2^100: every divisor and
// reciprocal is a normal number and the Markstein residuals of the quotients
// that decide a code are exact.
__device__ __forceinline__ bool scale_in_fast_range(float s_g) {
    return s_g >= 0x1p-80f && s_g <= 0x1p100f;
}

// ---------------------------------------------------------------------------
// E2M1 (FP4).  v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds binary32 to
// E2M1 with ties to the even code and saturates at +-6, keeping the sign;
// byte `sel` of `old` receives (code(a) | code(b) << 4).
// ---------------------------------------------------------------------------
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pack2(uint32_t old, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Codes for 8 consecutive bf16 values (4 packed words) of one block:
// element 2j in the low nibble of byte j.  d = RN(sf*s_g), r = RN(1/d).
// `fast` selects the Markstein quotient; otherwise correctly rounded division
// with a NaN quotient mapped to code 0.
__device__ __forceinline__ uint32_t quantize8f(const float v[8], float d, float r, bool fast) {
    float q[8];
    if (fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = div_markstein(v[i], d, r);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float t = v[i] / d;
            q[i] = (t != t) ? 0.0f : t;
        }
    }
    uint32_t w = 0;
    w = fp4_pack2<0>(w, q[0], q[1]);
    w = fp4_pack2<1>(w, q[2], q[3]);
    w = fp4_pack2<2>(w, q[4], q[5]);
    w = fp4_pack2<3>(w, q[6], q[7]);
    return w;
}

__device__ __forceinline__ uint32_t quantize8(const uint32_t y[4], float d, float r, bool fast) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_lo(y[j]);
        v[2 * j + 1] = bf16_hi(y[j]);
    }
    return quantize8f(v, d, r, fast);
}

// Everything one block needs after its maximum is known.
struct BlockQ {
    uint32_t sf;    // E4M3 code
    float d;        // RN(sf * s_g)
    float r;        // RN(1/d)
    bool fast;      // Markstein path valid
    uint32_t keep;  // 0 when the block is all-zero output (sf 0 or NaN code)
};

__device__ __forceinline__ BlockQ block_setup(uint32_t amax_bits16, float s_g, float rg, bool sg_fast) {
    BlockQ b;
    float a16 = __uint_as_float(amax_bits16 << 16);
    bool finite = amax_bits16 < 0x7F80u;
    b.fast = sg_fast && finite;
    b.sf = b.fast ? block_scale_fast(a16, s_g, rg) : block_scale_slow(a16, s_g);
    b.d = e4m3_value(b.sf) * s_g;
    b.r = 1.0f / b.d;  // correctly rounded
    b.keep = (b.sf == 0u || b.sf == 0x7Fu) ? 0u : 0xFFFFFFFFu;
    return b;
}

// d = RN(e4m3(c) * s_g) and r = RN(1/d) for all 128 codes c, the values
// block_setup computes per block; built once per workgroup so that a block's
// divisor and reciprocal become one LDS read.
__device__ __forceinline__ void build_dr_table(float2* dr, float s_g) {
    for (int c = threadIdx.x; c < 128; c += blockDim.x) {
        const float d = e4m3_value((uint32_t)c) * s_g;
        dr[c] = make_float2(d, 1.0f / d);
    }
    __syncthreads();
}

// BOUNDED: the block maximum is at most the maximum s_g was taken from
// (block_scale_bounded).  A tensor scale in the fast range then also means
// that maximum, and so every block, is finite: the choice of path is the same
// for every block of the launch.
template <bool BOUNDED = false>
__device__ __forceinline__ BlockQ block_setup_tab(uint32_t amax_bits16, float s_g, float rg, bool sg_fast,
                                                  const float2* dr) {
    BlockQ b;
    float a16 = __uint_as_float(amax_bits16 << 16);
    b.fast = BOUNDED ? sg_fast : sg_fast && amax_bits16 < 0x7F80u;
    if (!b.fast)
        b.sf = block_scale_slow(a16, s_g);
    else if constexpr (BOUNDED)
        b.sf = block_scale_bounded(a16, s_g, rg);
    else
        b.sf = block_scale_fast(a16, s_g, rg);
    const float2 t = dr[b.sf];
    b.d = t.x;
    b.r = t.y;
    b.keep = (b.sf == 0u || b.sf == 0x7Fu) ? 0u : 0xFFFFFFFFu;
    return b;
}

// Packed per-half maximum of two words of two uint16 each (v_pk_max_u16).
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a);
    u16x2 y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// |y| as bf16 magnitude bits for two packed values.  As unsigned integers these
// order finite magnitudes like the values and rank Inf and NaN above them.
__device__ __forceinline__ uint32_t mag2(uint32_t y2) { return y2 & 0x7FFF7FFFu; }

// Running packed maximum of magnitudes -> one 16-bit maximum.
__device__ __forceinline__ uint32_t fold_max(uint32_t m2) {
    uint32_t lo = m2 & 0xFFFFu, hi = m2 >> 16;
    return lo > hi ? lo : hi;
}

}  // namespace nvfp4
