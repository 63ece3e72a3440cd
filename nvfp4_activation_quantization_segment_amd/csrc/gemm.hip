// NVFP4 block-scaled GEMM for gfx950:  out = bf16(alpha * A W^T).
//
// Operation ("FC2 NVFP4 Library Scheduling", Exact Operation): packed
// activation rows [M,K] against packed weight rows [N,K], giving BF16 [M,N],
// FP32 accumulation, alpha = activation tensor scale * weight tensor scale
// applied before the BF16 conversion ("NVFP4 Streaming Design", P0).
//
// Decode.  Every E2M1 value times an E4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16; products of two such fp16
// values are exact in fp32.  The MFMA path is therefore f16 (same dense rate
// as bf16 on gfx950) with exact operands; only the fp32 accumulation order
// differs from an exact dot product.  A nibble pair decodes with one
// v_cvt_scalef32_pk_f16_fp4 (scale 256, a power of two, which the
// instruction applies exactly) followed by one v_pk_mul_f16 by the block
// scale as fp16 times 2^-8; v_cvt_scalef32_pk_f16_fp8 converts two scale
// bytes to those fp16 values at once, exactly, subnormals included, with the
// sign bit and the NaN code read as E4M3FN defines them.
//
// Tiling.  A workgroup of 8 waves (two per SIMD) computes a 256x256 output
// tile; each wave a 128(M) x 64(N) sub-tile as 4x2 v_mfma_f32_32x32x16_f16
// tiles with 128 fp32 accumulators per lane.  Every packed element is decoded
// once per workgroup into double-buffered fp16 tiles in LDS (256 rows x 64 per
// operand, row stride 144 bytes so that the 32 rows one MFMA fragment reads
// fall on distinct bank groups); the waves then read their fragments with
// 16-byte LDS loads.  The MFMA A operand is the weight (rows n) and the B
// operand the activation (rows m), so each lane's accumulators hold four
// consecutive n of one m and the epilogue stores 8 contiguous bytes.
//
// Global loads.  Waves 0-3 stage activation rows and waves 4-7 weight rows, 64
// rows per wave.  Lanes 2r and 2r+1 load the two 16-byte halves of one row's
// 32-byte K step, so a load instruction touches 32 rows rather than 64, and
// block scales are fetched for four K steps at a time (16 bytes per row).
// Measured on the projection shapes this halves the L1 accesses and L2
// requests of a one-row-per-lane layout, whose vector memory path was close to
// saturation; the energy saved shows up as clock under the power limit.  The
// loads are raw buffer loads: the operand's descriptor and the K-step offset
// are wave-uniform scalars and each lane's row offset is fixed, so the K loop
// spends no VALU instruction on addresses (the chip is power-limited under
// this kernel and every VALU instruction costs clock; measured 0.9% faster
// than 64-bit address arithmetic per load).
//
// Waves of tiles.  Tiles run in waves of one workgroup per CU.  With a
// workspace, a last wave that would leave most CUs idle is computed instead as
// several K ranges per tile (gemm_plan); the pieces store fp32 partial sums and
// gemm_finalize_kernel adds them in K order before the alpha and the bf16
// rounding.
#include <type_traits>

#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 64, kWM = 128, kWN = 64;
// Workgroup slots of one wave over the chip (256 CUs, one 512-thread workgroup each).
constexpr int kWaveSlots = 256;

// The E4M3 scales in bytes hb and hb+1 of a scale word, as two fp16 equal to
// sf * 2^-8 (v_cvt_scalef32_pk_f16_fp8: an exact conversion, subnormals
// included, with the power-of-two scale applied exactly).
__device__ __forceinline__ f16x2 sf_pair(uint32_t word, int hb) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word >> (8 * hb), 0x1p-8f, false);
}

// 8 nibbles (element 2i in the low nibble of byte i) times the block scale
// s (the same fp16 in both halves).
__device__ __forceinline__ f16x8 decode8(uint32_t w, f16x2 s) {
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
    return (f16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// LDS tiles: decoded fp16 [256 rows][64 k] per operand, row stride 72 halves
// (144 bytes: 16 bytes of padding make the 32 rows read by one MFMA fragment
// fall on distinct bank groups), two stages.
constexpr int kLDK = kBK + 8;
constexpr int kTileHalves = kBM * kLDK;  // per operand per stage
constexpr int kLdsBytes = 2 /*stages*/ * 2 /*operands*/ * kTileHalves * 2;

// One K step of the thread's two half rows: 32 nibbles each.
struct RowPack {
    uint4 q[2];
};
// Block scales of the thread's two rows for a group of 4 K steps: word j of
// s[i] holds the 4 scales of row i in step 4g+j.
struct ScaleGrp {
    uint4 s[2];
};

// Raw buffer resource over an operand: base and per-lane offsets of the
// loads below are 32-bit, the descriptor lives in scalar registers, and the
// K-step offset is a scalar operand of the load, so a load takes no VALU
// address arithmetic.  The range is the whole 32-bit offset space (every
// offset the kernel forms is below 2^32).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const uint8_t* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, 0xFFFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ RowPack load_row(__amdgpu_buffer_rsrc_t q, uint32_t soff, uint32_t q0, uint32_t q1) {
    RowPack r;
    r.q[0] = buf_load16(q, q0, soff);
    r.q[1] = buf_load16(q, q1, soff);
    return r;
}

// Scales of group g.  With SC4 (scale rows and base pointers 16-byte aligned,
// K a multiple of 256) one 16-byte load per row; otherwise four 4-byte loads,
// steps past the last clamped to it.
template <bool SC4>
__device__ __forceinline__ ScaleGrp load_grp(__amdgpu_buffer_rsrc_t sf, uint32_t s0, uint32_t s1, int g, int nit) {
    ScaleGrp r;
    if (SC4) {
        r.s[0] = buf_load16(sf, s0, 16u * g);
        r.s[1] = buf_load16(sf, s1, 16u * g);
    } else {
        uint32_t w[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int st = 4 * g + j < nit ? 4 * g + j : nit - 1;
            w[0][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(sf, (int)s0, (int)(4u * st), 0);
            w[1][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(sf, (int)s1, (int)(4u * st), 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) r.s[i] = (uint4){w[i][0], w[i][1], w[i][2], w[i][3]};
    }
    return r;
}

// Decode part p (row p>>1, words 2(p&1) and 2(p&1)+1: the 16 values of one
// block) of the thread's staged half rows into LDS: two 16-byte stores.  sp[i]
// holds row i's two block scales of the step for this thread's half row.
__device__ __forceinline__ void store_part(const RowPack& r, const f16x2 (&sp)[2], int p, _Float16* dst0,
                                           _Float16* dst1) {
    const int i = p >> 1, wp = p & 1;
    const f16x2 s2 = {sp[i][wp], sp[i][wp]};
    _Float16* dst = i == 0 ? dst0 : dst1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int w = 2 * wp + u;
        *reinterpret_cast<f16x8*>(dst + 8 * w) = decode8(word_of(r.q[i], w), s2);
    }
}

// Per-thread staging geometry.
struct Stage {
    __amdgpu_buffer_rsrc_t qr;  // packed rows of the thread's operand
    __amdgpu_buffer_rsrc_t sr;  // their scales
    uint32_t q0, q1;    // byte offsets of the two half rows (step 0)
    uint32_t s0, s1;    // byte offsets of the two scale rows
    int dop;            // LDS operand index: 0 activation, 2 weight
    int d0, d1;         // LDS offsets (halves) of the two decoded half rows
    int hb;             // 2 * (half of the row this thread holds)
};

// K step `it` on LDS buffer CUR, in four phases (one per 16-wide K slice j):
// read the fragments of slice j+1, decode one part of this thread's share of
// step it+1 into the other buffer, and issue the 8 MFMAs of slice j.  CUR is a
// template parameter so that both buffers' offsets are constants and the reads
// of one buffer and the writes of the other are visibly independent.  The
// packed data of step it+2 (and, with LOADG, the scale group after the current
// one) is fetched at the start of the step.  SW selects the scale word of step
// it+1: word SW of the current group, or word 0 of the next group for SW == 4.
template <int CUR, int SW, bool LOADG, bool SC4>
__device__ __forceinline__ void k_step(_Float16* __restrict__ lds, f32x16 (&acc)[2][4], RowPack& ra,
                                       ScaleGrp& gc, ScaleGrp& gn, const Stage& st, int next_stage,
                                       int next_grp, int nit, int wrow0, int arow0, int h) {
    const _Float16* cA = lds + CUR * kTileHalves;
    const _Float16* cW = lds + (2 + CUR) * kTileHalves;
    _Float16* dst0 = lds + (st.dop + (CUR ^ 1)) * kTileHalves + st.d0;
    _Float16* dst1 = lds + (st.dop + (CUR ^ 1)) * kTileHalves + st.d1;
    const ScaleGrp& gs = SW < 4 ? gc : gn;
    const f16x2 sp[2] = {sf_pair(word_of(gs.s[0], SW & 3), st.hb), sf_pair(word_of(gs.s[1], SW & 3), st.hb)};
    const RowPack na = load_row(st.qr, 32u * next_stage, st.q0, st.q1);
    if (LOADG) gn = load_grp<SC4>(st.sr, st.s0, st.s1, next_grp, nit);
    f16x8 wf[2][2], af[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) wf[0][i] = *reinterpret_cast<const f16x8*>(cW + (wrow0 + 32 * i) * kLDK + 8 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = *reinterpret_cast<const f16x8*>(cA + (arow0 + 32 * i) * kLDK + 8 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int b = j & 1;
        if (j < 3) {
            const int kk = 16 * (j + 1) + 8 * h;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                wf[b ^ 1][i] = *reinterpret_cast<const f16x8*>(cW + (wrow0 + 32 * i) * kLDK + kk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[b ^ 1][i] = *reinterpret_cast<const f16x8*>(cA + (arow0 + 32 * i) * kLDK + kk);
        }
        store_part(ra, sp, j, dst0, dst1);
        // Four MFMAs in a row share one weight fragment, and the activation
        // fragments run 0..3 then 3..0, so that consecutive instructions
        // change as few operands as possible: under the power limit fewer
        // operand changes mean a higher clock (measured 0.8% for keeping the
        // A operand, 0.2-0.5% more for the reversed second row).
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = i ? 3 - kk : kk;
                acc[i][k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[b][i], af[b][k], acc[i][k], 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
    }
    ra = na;
    if (SW == 4) gc = gn;
    __syncthreads();
}

// Output tile of logical tile index `logical`: tiles are walked in groups of
// 4 M-tiles (all N-tiles of a group before the next group), so that the
// workgroups resident on one XCD share activation and weight rows in L2.
__device__ __forceinline__ void tile_coords(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
    constexpr int GM = 4;
    const int gsz = GM * tiles_n;
    const int first_m = (logical / gsz) * GM;
    const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    tm = first_m + (logical % gsz) % gm;
    tn = (logical % gsz) / gm;
}

// Residual epilogue ("NVFP4 Streaming Design", P4: the GEMM result rounded to
// BF16, scaled by the gate, added to the residual, rounded again): for two
// packed outputs o2, gates g2 and residuals r2, bf16(r + bf16(g * o)); the
// product of two bf16 values is exact in binary32.
__device__ __forceinline__ uint32_t gate_residual2(uint32_t o2, uint32_t g2, uint32_t r2) {
    const float pa = round_bf16(bf16_lo(g2) * bf16_lo(o2)), pb = round_bf16(bf16_hi(g2) * bf16_hi(o2));
    return pack_bf16x2(bf16_lo(r2) + pa, bf16_hi(r2) + pb);
}

// Gate row of output row m (segments are contiguous row ranges).
__device__ __forceinline__ const uint16_t* gate_row(const GemmArgs& a, int m) {
    int s = 0;
    while (s + 1 < a.nseg && m >= a.row_start[s + 1]) ++s;
    return a.gate + (int64_t)s * a.ld_gate;
}

// The 8-byte store of 4 outputs at (m, n), through the epilogue when enabled.
__device__ __forceinline__ void store_out4(const GemmArgs& a, int m, int n, uint2 v) {
    if (a.epi) {
        const uint2 g = *reinterpret_cast<const uint2*>(gate_row(a, m) + n);
        const uint2 r = *reinterpret_cast<const uint2*>(a.residual + (int64_t)m * a.ldr + n);
        v.x = gate_residual2(v.x, g.x, r.x);
        v.y = gate_residual2(v.y, g.y, r.y);
    }
    *reinterpret_cast<uint2*>(a.out + (int64_t)m * a.ldo + n) = v;
}

// One launch's share of the output tiles.  The main launch computes tiles
// [0, tiles) over all of K; a split launch computes `tiles` tail tiles from
// tile_base on, each as ksplit K ranges of ks steps, and stores fp32 partial
// sums for gemm_finalize_kernel.
template <bool SC4, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void
gemm_kernel(GemmArgs a, GemmPart p) {
    __shared__ __attribute__((aligned(16))) _Float16 lds[kLdsBytes / 2];

    // Tile order: in the main launch each XCD (workgroups are dealt
    // round-robin over 8) takes a contiguous range of logical tiles.
    const int bid = blockIdx.x;
    int logical, k0 = 0, nit = a.K / kBK, split = 0, tail = 0;
    if (!SPLIT) {
        const int per = p.tiles / 8;
        logical = (bid < per * 8) ? (bid % 8) * per + bid / 8 : bid;
    } else {
        tail = bid / p.ksplit;
        split = bid - tail * p.ksplit;
        logical = p.tile_base + tail;
        k0 = split * p.ks;
        nit = nit - k0 < p.ks ? nit - k0 : p.ks;
    }
    int tm, tn;
    tile_coords(logical, p.tiles_m, p.tiles_n, tm, tn);

    const int tid = threadIdx.x;
    // the wave index through readfirstlane: wave-uniform values (the operand
    // base pointers, the K-step offsets) then live in scalar registers, and
    // every global load takes a scalar base plus a fixed per-lane offset
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int h = lane >> 5, l32 = lane & 31;
    // The two waves of a SIMD (w and w+4) run the same instruction stream;
    // giving one of them a higher issue priority breaks the tie, so one runs
    // ahead and the other fills its gaps (measured +2-3% over equal priority).
    if (wave < 4) __builtin_amdgcn_s_setprio(2);
    const uint32_t Kb = (uint32_t)a.K >> 1, Ks = (uint32_t)a.K >> 4;

    // Staging role: lane 2r+sh of wave w holds half sh of rows r and r+32 of
    // the 64 rows (w & 3) * 64 .. of the activation tile (w < 4) or the weight
    // tile (w >= 4); rows past the end are clamped to the last row.
    Stage st;
    const bool is_a = wave < 4;
    st.qr = operand_rsrc(is_a ? a.qa : a.qw);
    st.sr = operand_rsrc(is_a ? a.sfa : a.sfw);
    const int sh = lane & 1;
    const int lr = (wave & 3) * 64 + (lane >> 1);
    {
        uint32_t qo[2], so[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int row;
            if (is_a) {
                row = tm * kBM + lr + 32 * i;
                row = row < a.M_pad ? row : a.M_pad - 1;
            } else {
                row = tn * kBN + lr + 32 * i;
                row = row < a.N ? row : a.N - 1;
            }
            qo[i] = (uint32_t)row * Kb + 16u * sh + 32u * (uint32_t)k0;
            so[i] = (uint32_t)row * Ks + 4u * (uint32_t)k0;
        }
        st.q0 = qo[0];
        st.q1 = qo[1];
        st.s0 = so[0];
        st.s1 = so[1];
    }
    st.dop = is_a ? 0 : 2;
    st.d0 = lr * kLDK + 32 * sh;
    st.d1 = (lr + 32) * kLDK + 32 * sh;
    st.hb = 2 * sh;

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = (f32x16){0};
    const int wrow0 = wn * kWN + l32;
    const int arow0 = wm * kWM + l32;
    const int ngrp = (nit + 3) / 4;
    const int lastst = nit - 1;

    // Prologue: decode step 0 into buffer 0, fetch step 1.
    RowPack ra = load_row(st.qr, 0u, st.q0, st.q1);
    ScaleGrp gc = load_grp<SC4>(st.sr, st.s0, st.s1, 0, nit), gn = gc;
    {
        const f16x2 sp[2] = {sf_pair(gc.s[0].x, st.hb), sf_pair(gc.s[1].x, st.hb)};
#pragma unroll
        for (int p = 0; p < 4; ++p)
            store_part(ra, sp, p, lds + st.dop * kTileHalves + st.d0, lds + st.dop * kTileHalves + st.d1);
    }
    {
        const uint32_t s1 = nit > 1 ? 1 : 0;
        ra = load_row(st.qr, 32u * s1, st.q0, st.q1);
    }
    __syncthreads();

    // Step it decodes step it+1 (scale word (it+1) % 4) and fetches the data of
    // step it+2; the step with it % 4 == 2 also fetches the next scale group.
    // Fetches past the last step are clamped to it and never used.
    int it = 0;
#define NVFP4_KSTEP(C, SW, LG, NS)                                                                        \
    k_step<C, SW, LG, SC4>(lds, acc, ra, gc, gn, st, (NS) < lastst ? (NS) : lastst,                      \
                           (it >> 2) + 1 < ngrp ? (it >> 2) + 1 : ngrp - 1, nit, wrow0, arow0, h)
    for (; it + 4 <= nit - 1; it += 4) {
        NVFP4_KSTEP(0, 1, false, it + 2);
        NVFP4_KSTEP(1, 2, false, it + 3);
        NVFP4_KSTEP(0, 3, true, it + 4);
        NVFP4_KSTEP(1, 4, false, it + 5);
    }
    {
        const int rem = nit - 1 - it;  // 0..3 decoding steps left, uniform
        if (rem > 0) NVFP4_KSTEP(0, 1, false, it + 2);
        if (rem > 1) NVFP4_KSTEP(1, 2, false, it + 3);
        if (rem > 2) NVFP4_KSTEP(0, 3, true, it + 4);
        it += rem;
    }
#undef NVFP4_KSTEP

    // Last step: MFMAs only.
    {
        const _Float16* cA = lds + (it & 1) * kTileHalves;
        const _Float16* cW = lds + (2 + (it & 1)) * kTileHalves;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = 16 * j + 8 * h;
            f16x8 wf[2], af[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) wf[i] = *reinterpret_cast<const f16x8*>(cW + (wrow0 + 32 * i) * kLDK + kk);
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const f16x8*>(cA + (arow0 + 32 * i) * kLDK + kk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k = i ? 3 - kk : kk;
                    acc[i][k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[i], af[k], acc[i][k], 0, 0, 0);
                }
        }
    }

    if (SPLIT) {
        // fp32 partial sums: slot (tail, split), then wave, accumulator quad
        // (4 consecutive registers = 4 consecutive n), lane; each float4
        // store of a wave writes 1 KB contiguously.
        float4* dst = reinterpret_cast<float4*>(p.partial) +
                      ((size_t)(tail * p.ksplit + split) * 8 + wave) * (32 * 64) + lane;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16& c = acc[i][k];
                    // non-temporal: the next producer pass otherwise waits on these
                    // lines' write-back from the memory-side cache
                    store_nt(reinterpret_cast<uint4*>(&dst[((i * 4 + k) * 4 + q) * 64]),
                             make_uint4(__float_as_uint(c[4 * q]), __float_as_uint(c[4 * q + 1]),
                                        __float_as_uint(c[4 * q + 2]), __float_as_uint(c[4 * q + 3])));
                }
        return;
    }

    // Epilogue: alpha = RN(s_a * s_w) applied in fp32, then bf16 (nearest-even).
    const float alpha = a.a_scale[0] * a.w_scale[0];
    const bool rows16 = ((reinterpret_cast<uintptr_t>(a.out) & 15) == 0 && (a.ldo & 7) == 0) &&
                        (!a.epi || (((reinterpret_cast<uintptr_t>(a.gate) | reinterpret_cast<uintptr_t>(a.residual)) &
                                     15) == 0 &&
                                    ((a.ld_gate | a.ldr) & 7) == 0));
    if (rows16) {
        // Each wave stages its 128 x 64 bf16 sub-tile in LDS (rows of 144
        // bytes) and writes it back as whole 128-byte rows, eight lanes per
        // row, with non-temporal stores: the output (up to 1.6 GB) then leaves
        // no dirty lines in the memory-side cache, which would slow the
        // kernel that runs next (the following producer pass reads 0.4-2 GB).
        constexpr int kRowB = 144;
        char* wl = reinterpret_cast<char*>(lds) + wave * (kWM * kRowB);
        __syncthreads();  // the last step's fragment reads are done
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16& c = acc[i][k];
                    uint2 v;
                    v.x = pack_bf16x2(c[4 * q + 0] * alpha, c[4 * q + 1] * alpha);
                    v.y = pack_bf16x2(c[4 * q + 2] * alpha, c[4 * q + 3] * alpha);
                    *reinterpret_cast<uint2*>(wl + (k * 32 + l32) * kRowB + (i * 32 + 8 * q + 4 * h) * 2) = v;
                }
        __syncthreads();
        const int n = tn * kBN + wn * kWN + (lane & 7) * 8;
        const int m0 = tm * kBM + wm * kWM + (lane >> 3);
        if (n < a.N && !a.epi) {
#pragma unroll
            for (int it = 0; it < kWM / 8; ++it) {
                const int m = m0 + 8 * it;
                if (m < a.M) {
                    const uint4 v =
                        *reinterpret_cast<const uint4*>(wl + (8 * it + (lane >> 3)) * kRowB + (lane & 7) * 16);
                    store_nt(reinterpret_cast<uint4*>(a.out + (int64_t)m * a.ldo + n), v);
                }
            }
        } else if (n < a.N) {
            // Residual epilogue: the lane's residual loads issued 8 rows at a
            // time (rows past M clamped to the last row, never stored; 8
            // rather than all 16, which would not fit the registers left and
            // spilled), and one gate vector when the wave's 128 rows lie in
            // one segment, so that the load latency is paid twice rather than
            // once per row.
            const int wfirst = tm * kBM + wm * kWM;
            const int wlast = wfirst + kWM - 1 < a.M - 1 ? wfirst + kWM - 1 : a.M - 1;
            const uint16_t* g_first = gate_row(a, wfirst < a.M ? wfirst : a.M - 1);
            const bool one_gate = g_first == gate_row(a, wlast);
            const uint4 g_wave = *reinterpret_cast<const uint4*>(g_first + n);
            // The choice of gate is a wave-uniform branch around the whole
            // loop: a per-row select between g_wave and a load would become a
            // load through a selected pointer, with g_wave put on the stack.
            const auto rows = [&](auto one) {
                constexpr int kBatch = 8;
#pragma unroll
                for (int b0 = 0; b0 < kWM / 8; b0 += kBatch) {
                    uint4 res[kBatch];
#pragma unroll
                    for (int it = 0; it < kBatch; ++it) {
                        const int m = m0 + 8 * (b0 + it) < a.M ? m0 + 8 * (b0 + it) : a.M - 1;
                        res[it] = *reinterpret_cast<const uint4*>(a.residual + (int64_t)m * a.ldr + n);
                    }
#pragma unroll
                    for (int it = 0; it < kBatch; ++it) {
                        const int m = m0 + 8 * (b0 + it);
                        if (m < a.M) {
                            uint4 v = *reinterpret_cast<const uint4*>(wl + (8 * (b0 + it) + (lane >> 3)) * kRowB +
                                                                      (lane & 7) * 16);
                            const uint4 g = decltype(one)::value
                                                ? g_wave
                                                : *reinterpret_cast<const uint4*>(gate_row(a, m) + n);
                            v.x = gate_residual2(v.x, g.x, res[it].x);
                            v.y = gate_residual2(v.y, g.y, res[it].y);
                            v.z = gate_residual2(v.z, g.z, res[it].z);
                            v.w = gate_residual2(v.w, g.w, res[it].w);
                            store_nt(reinterpret_cast<uint4*>(a.out + (int64_t)m * a.ldo + n), v);
                        }
                    }
                }
            };
            if (one_gate)
                rows(std::true_type{});
            else
                rows(std::false_type{});
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int m = tm * kBM + wm * kWM + k * 32 + l32;
        if (m >= a.M) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = tn * kBN + wn * kWN + i * 32 + 8 * q + 4 * h;
                if (n >= a.N) continue;
                const f32x16& c = acc[i][k];
                uint2 v;
                v.x = pack_bf16x2(c[4 * q + 0] * alpha, c[4 * q + 1] * alpha);
                v.y = pack_bf16x2(c[4 * q + 2] * alpha, c[4 * q + 3] * alpha);
                store_out4(a, m, n, v);
            }
        }
    }
}

// Sums the ksplit partials of each tail tile in split order, applies alpha
// and writes bf16 with the main epilogue's layout.  One 64-thread workgroup
// per (tail tile, wave, 32-row group k): 8 output quads per lane, the partial
// loads of a quad issued together.
constexpr int kMaxSplit = 16;
__global__ __launch_bounds__(64) void gemm_finalize_kernel(GemmArgs a, GemmPart p) {
    const int tail = blockIdx.x >> 5;
    const int wave = (blockIdx.x >> 2) & 7;
    const int k = blockIdx.x & 3;
    int tm, tn;
    tile_coords(p.tile_base + tail, p.tiles_m, p.tiles_n, tm, tn);
    const int lane = threadIdx.x;
    const int wm = wave >> 2, wn = wave & 3;
    const int h = lane >> 5, l32 = lane & 31;
    const int m = tm * kBM + wm * kWM + k * 32 + l32;
    if (m >= a.M) return;
    const float alpha = a.a_scale[0] * a.w_scale[0];
    const size_t slot = (size_t)8 * 32 * 64;  // float4 per partial tile
    const float4* src = reinterpret_cast<const float4*>(p.partial) + (size_t)tail * p.ksplit * slot +
                        (size_t)wave * (32 * 64) + lane;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = tn * kBN + wn * kWN + i * 32 + 8 * q + 4 * h;
            if (n >= a.N) continue;
            const float4* pe = src + ((i * 4 + k) * 4 + q) * 64;
            float4 v[kMaxSplit];
#pragma unroll
            for (int sp = 0; sp < kMaxSplit; ++sp)
                if (sp < p.ksplit) v[sp] = pe[(size_t)sp * slot];
            float4 acc = v[0];
#pragma unroll
            for (int sp = 1; sp < kMaxSplit; ++sp)
                if (sp < p.ksplit) {
                    acc.x += v[sp].x;
                    acc.y += v[sp].y;
                    acc.z += v[sp].z;
                    acc.w += v[sp].w;
                }
            uint2 w;
            w.x = pack_bf16x2(acc.x * alpha, acc.y * alpha);
            w.y = pack_bf16x2(acc.z * alpha, acc.w * alpha);
            store_out4(a, m, n, w);
        }
    }
}

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K) {
    GemmPlan pl;
    pl.tiles_m = (int)((M + kBM - 1) / kBM);
    pl.tiles_n = (int)((N + kBN - 1) / kBN);
    const int T = pl.tiles_m * pl.tiles_n;
    const int nit = (int)(K / kBK);
    pl.full = T;
    pl.tail = 0;
    pl.ksplit = 1;
    pl.ks = nit;
    pl.workspace_bytes = 0;
    // A last wave of at most a third of the workgroup slots is split along K
    // into as many pieces as fill the slots, each at least 4 K steps and a
    // multiple of 4 (whole scale groups).
    const int R = T % kWaveSlots;
    if (R == 0 || 3 * R > kWaveSlots) return pl;
    int S = kWaveSlots / R;
    if (S > kMaxSplit) S = kMaxSplit;
    if (S > nit / 4) S = nit / 4;
    if (S < 2) return pl;
    int ks = (nit + S - 1) / S;
    ks = (ks + 3) / 4 * 4;
    S = (nit + ks - 1) / ks;
    if (S < 2) return pl;
    pl.full = T - R;
    pl.tail = R;
    pl.ksplit = S;
    pl.ks = ks;
    pl.workspace_bytes = (size_t)R * S * 8 * 32 * 64 * sizeof(float4);
    return pl;
}

static bool scales_16b(const GemmArgs& a) {
    // 16-byte scale-group loads need every scale row and both base pointers
    // 16-byte aligned, i.e. K/16 a multiple of 16.
    return (a.K >> 4) % 16 == 0 &&
           ((reinterpret_cast<uintptr_t>(a.sfa) | reinterpret_cast<uintptr_t>(a.sfw)) & 15) == 0;
}

template <bool SC4>
static hipError_t launch_all(const GemmArgs& a, const GemmPlan& pl, float* workspace, hipStream_t s) {
    GemmPart p;
    p.tiles_m = pl.tiles_m;
    p.tiles_n = pl.tiles_n;
    p.tile_base = 0;
    p.tiles = pl.full;
    p.ksplit = 1;
    p.ks = pl.ks;
    p.partial = workspace;
    if (pl.full > 0)
        hipLaunchKernelGGL((gemm_kernel<SC4, false>), dim3(pl.full), dim3(512), 0, s, a, p);
    if (pl.tail > 0) {
        p.tile_base = pl.full;
        p.tiles = pl.tail;
        p.ksplit = pl.ksplit;
        hipLaunchKernelGGL((gemm_kernel<SC4, true>), dim3(pl.tail * pl.ksplit), dim3(512), 0, s, a, p);
        hipLaunchKernelGGL(gemm_finalize_kernel, dim3(pl.tail * 32), dim3(64), 0, s, a, p);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, float* workspace, bool split, hipStream_t s) {
    GemmPlan pl = gemm_plan(a.M, a.N, a.K);
    if (!split || !workspace) {
        pl.full = pl.tiles_m * pl.tiles_n;
        pl.tail = 0;
    }
    return scales_16b(a) ? launch_all<true>(a, pl, workspace, s) : launch_all<false>(a, pl, workspace, s);
}

}  // namespace nvfp4
