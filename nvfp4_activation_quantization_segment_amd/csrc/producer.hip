// NVFP4 activation producer kernels for gfx950.
//
// Two passes over the BF16 input, as the exact two-phase design requires
// ("NVFP4 Streaming Design", Numerical Constraint: no tile can be packed
// before the global reduction completes; "NVFP4 Modulation Producer Fusion",
// Dataflow: read the normalized input, reproduce the BF16 modulation and
// reduce |y| without writing y; read it again and write QDATA/SFA into
// caller-owned buffers).
//
// Layout of the work: in pass 1 one thread owns one 8-column chunk (16 bytes
// of bf16), in pass 2 one 16-column block (32 bytes), of every row its
// workgroup visits.  A workgroup spans every chunk of a row (blockDim = chunks
// per row rounded up to 64, a thread taking several chunks when a row has more
// than 1024), so each row is read with contiguous 16-byte loads and the
// per-column bf16(scale+1) and shift stay in registers.  Workgroups take rows
// grid-stride, so the rows in flight form one compact window of the tensor.
#include <type_traits>

#include "nvfp4_device.h"
#include "internal.h"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// Raises the workgroup's shared threshold word (float bits; the values are
// non-negative or NaN, which order as their bit patterns) with this wave's
// largest mf and returns the new value, the same in every lane.
__device__ __forceinline__ float raise_threshold(uint32_t* word, float mf) {
    const uint32_t w = wave_max_u32(__float_as_uint(mf));
    uint32_t v = 0;
    if ((threadIdx.x & 63) == 0) v = atomicMax(word, w);
    v = (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
    return __uint_as_float(v > w ? v : w);
}

// Workgroup maximum of a 16-bit magnitude, then the grid-level finish: one
// atomic max per workgroup; the last workgroup to take a ticket turns the
// maximum into the tensor scale and returns the workspace to zero.
//
// Only atomic read-modify-writes touch the two workspace words, and device-
// scope RMWs on one location are totally ordered, so no cache-wide fence is
// needed (an agent-scope fence here writes back and invalidates the XCD's L2
// once per workgroup, which dominated the pass).  Each workgroup consumes the
// value returned by its max before taking its ticket, so the max has been
// performed first; the last workgroup reads the maximum with an RMW after
// every other ticket, hence after every other max.
__device__ __forceinline__ uint32_t atomic_max_dev(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_add_dev(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ void reduce_and_finish(uint32_t m16, uint32_t* ws, float* tensor_scale, float* amax_out) {
    __shared__ uint32_t red[16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    m16 = wave_max_u32(m16);
    if (lane == 0) red[w] = m16;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t mm = 0;
        const int nw = (blockDim.x + 63) >> 6;
        for (int i = 0; i < nw; ++i) mm = red[i] > mm ? red[i] : mm;
        const uint32_t prev = atomic_max_dev(&ws[0], mm);
        asm volatile("" ::"v"(prev) : "memory");  // the max is performed before the ticket
        const uint32_t ticket = atomic_add_dev(&ws[1], 1u);
        if (ticket == gridDim.x - 1) {
            const uint32_t bits = atomic_max_dev(&ws[0], 0u);
            const float amax = __uint_as_float(bits << 16);
            // s_g = amax / (6 * 448), or 1 when the tensor is all zero
            const float sg = (amax == 0.0f) ? 1.0f : amax / 2688.0f;
            tensor_scale[0] = sg;
            if (amax_out) amax_out[0] = amax;
            __hip_atomic_exchange(&ws[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_exchange(&ws[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// One block's output: its 8 QDATA bytes and its scale byte.
struct PackedBlock {
    uint2 w;
    uint32_t sf;
};

// QDATA with a non-temporal store (whole lines per wave), the scale byte with
// a plain one.
__device__ __forceinline__ void store_block(const PackedBlock& pb, uint8_t* __restrict__ q, uint8_t* __restrict__ sf) {
    store_nt(reinterpret_cast<uint2*>(q), pb.w);
    *sf = (uint8_t)pb.sf;
}

// One thread, one whole 16-value block given as 8 packed bf16 pairs: maximum,
// scale and codes (pack_block16_store also stores them for block b of a row).
template <bool BOUNDED = false>
__device__ __forceinline__ PackedBlock pack_block16(const uint32_t y[8], float s_g, float rg, bool sg_fast,
                                                    const float2* dr) {
    uint32_t m2 = mag2(y[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k) m2 = pk_max_u16(m2, mag2(y[k]));
    const BlockQ bq = block_setup_tab<BOUNDED>(fold_max(m2), s_g, rg, sg_fast, dr);
    PackedBlock pb;
    pb.w.x = quantize8(y, bq.d, bq.r, bq.fast) & bq.keep;
    pb.w.y = quantize8(y + 4, bq.d, bq.r, bq.fast) & bq.keep;
    pb.sf = bq.sf;
    return pb;
}

template <bool BOUNDED = false>
__device__ __forceinline__ void pack_block16_store(const uint32_t y[8], float s_g, float rg, bool sg_fast,
                                                   const float2* dr, uint8_t* __restrict__ qrow,
                                                   uint8_t* __restrict__ srow, int b) {
    store_block(pack_block16<BOUNDED>(y, s_g, rg, sg_fast, dr), qrow + 8 * b, srow + b);
}

// ---------------------------------------------------------------------------
// Modulation producer
// ---------------------------------------------------------------------------
struct ColParams {
    float s1[8];
    float sh[8];
};

__device__ __forceinline__ void load_cols(const SegParams& seg, int s, int c, ColParams& cp) {
    const uint4 sc = ld16(seg.scale + (int64_t)s * seg.ld + 8 * c);
    const uint4 sh = ld16(seg.shift + (int64_t)s * seg.ld + 8 * c);
    const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
    const uint32_t shw[4] = {sh.x, sh.y, sh.z, sh.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        cp.s1[2 * j] = mod_scale1((uint16_t)(scw[j] & 0xFFFF));
        cp.s1[2 * j + 1] = mod_scale1((uint16_t)(scw[j] >> 16));
        cp.sh[2 * j] = bf16_lo(shw[j]);
        cp.sh[2 * j + 1] = bf16_hi(shw[j]);
    }
}

__device__ __forceinline__ void modulate8(const uint4 xv, const ColParams& cp, uint32_t y[4]) {
    y[0] = modulate2(xv.x, cp.s1[0], cp.s1[1], cp.sh[0], cp.sh[1]);
    y[1] = modulate2(xv.y, cp.s1[2], cp.s1[3], cp.sh[2], cp.sh[3]);
    y[2] = modulate2(xv.z, cp.s1[4], cp.s1[5], cp.sh[4], cp.sh[5]);
    y[3] = modulate2(xv.w, cp.s1[6], cp.s1[7], cp.sh[6], cp.sh[7]);
}

// Segment of row r: segments are contiguous row ranges; rows visit in order,
// so the caller keeps the current segment and its end and advances rarely.
__device__ __forceinline__ int seg_advance(const SegParams& seg, int64_t r, int s) {
    while (r >= seg.row_start[s + 1]) ++s;
    return s;
}

// Running maximum of the magnitudes of the unrounded modulation sums of 8
// columns (NaN once any is NaN); see mod16_max.
__device__ __forceinline__ float mod8_max(const uint4& xv, const ColParams& cp, float m) {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float sa = round_bf16(bf16_lo(xw[j]) * cp.s1[2 * j]) + cp.sh[2 * j];
        const float sb = round_bf16(bf16_hi(xw[j]) * cp.s1[2 * j + 1]) + cp.sh[2 * j + 1];
        m = __builtin_elementwise_maximum(
            m, __builtin_elementwise_maximum(__builtin_fabsf(sa), __builtin_fabsf(sb)));
    }
    return m;
}

// Pass 1 of the modulation producer (and of the plain quantizer).  Rows are
// assigned grid-stride (workgroup b takes rows b, b+G, b+2G, ...), so the
// workgroups resident at any moment read one compact window of the tensor
// that sweeps through it, which is what the memory system streams best.
// PLAIN: y = x (seg is not read).  EXACT: the
// maximum of the rounded y's bf16 magnitude bits; otherwise the maximum of the
// unrounded sums, whose bf16 rounding is the same value (the kernel reruns the
// exact form for a thread that met a NaN, so that the largest NaN bit pattern
// is found as the exact form finds it).
template <bool PLAIN, bool EXACT>
__device__ __forceinline__ uint32_t modulate_absmax_rows(const uint16_t* __restrict__ x, const RowGeo& g,
                                                         const SegParams& seg, float& mf) {
    const int64_t G = gridDim.x;
    uint32_t m2 = 0;
    for (int j = 0; j < g.J; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c >= g.C8) break;
        int64_t r = blockIdx.x;
        int s = seg_advance(seg, r < g.M ? r : 0, 0);
        int64_t seg_end = seg.row_start[s + 1];  // rows only increase: one compare per row
        ColParams cp;
        if (!PLAIN) load_cols(seg, s, c, cp);
        auto one = [&](const uint4& xv, int64_t rr) {
            if constexpr (PLAIN) {
                const uint32_t y[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(y[k]));
            } else {
                if (rr >= seg_end) {
                    s = seg_advance(seg, rr, s);
                    seg_end = seg.row_start[s + 1];
                    load_cols(seg, s, c, cp);
                }
                if constexpr (EXACT) {
                    uint32_t y[4];
                    modulate8(xv, cp, y);
#pragma unroll
                    for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(y[k]));
                } else {
                    mf = mod8_max(xv, cp, mf);
                }
            }
        };
        for (; r + 3 * G < g.M; r += 4 * G) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = ld16(x + (r + u * G) * g.ldx + 8 * c);
#pragma unroll
            for (int u = 0; u < 4; ++u) one(v[u], r + u * G);
        }
        for (; r < g.M; r += G) one(ld16(x + r * g.ldx + 8 * c), r);
    }
    return m2;
}

template <bool PLAIN>
__global__ __launch_bounds__(1024) void modulate_absmax_kernel(const uint16_t* __restrict__ x, RowGeo g,
                                                               SegParams seg, uint32_t* ws,
                                                               float* tensor_scale, float* amax_out) {
    float mf = 0.0f;
    uint32_t m;
    if constexpr (PLAIN) {
        m = fold_max(modulate_absmax_rows<true, true>(x, g, seg, mf));
    } else {
        modulate_absmax_rows<false, false>(x, g, seg, mf);
        if (mf == mf)
            m = __float_as_uint(round_bf16(mf)) >> 16;
        else
            m = fold_max(modulate_absmax_rows<false, true>(x, g, seg, mf));
    }
    reduce_and_finish(m, ws, tensor_scale, amax_out);
}

// Pass 2: one thread per 16-value block (two 16-byte loads per row), so the
// block scale is computed once.  Rows are walked last-to-first (grid-stride
// from the end), so the rows pass 1 read last, which are still in the
// memory-side cache, are read first.
template <bool PLAIN>
__global__ __launch_bounds__(1024) void modulate_pack_kernel(const uint16_t* __restrict__ x, RowGeo g,
                                                             SegParams seg, const float* tensor_scale,
                                                             uint8_t* __restrict__ qdata,
                                                             uint8_t* __restrict__ sfa, int reverse) {
    __shared__ float2 dr[128];
    const float s_g = tensor_scale[0];
    build_dr_table(dr, s_g);
    const bool sg_fast = scale_in_fast_range(s_g);
    const float rg = 1.0f / s_g;
    const int64_t G = gridDim.x;
    const int C16 = g.C8 >> 1;
    const int64_t qld = 8 * (int64_t)C16, sld = C16;
    // a workgroup iteration covers R rows: thread idx takes block idx % C16 of
    // row offset idx / C16 (R > 1 only when a row has at most 512 blocks)
    const int64_t GR = G * g.R;
    for (int j = 0; j < g.J; ++j) {
        const int idx = threadIdx.x + j * blockDim.x;
        const int rho = idx / C16;
        const int b = idx - rho * C16;
        if (rho >= g.R) break;
        // padding rows M .. rows_total-1 are zero
        for (int64_t r = g.M + (int64_t)blockIdx.x * g.R + rho; r < g.rows_total; r += GR) {
            store_nt(reinterpret_cast<uint2*>(qdata + r * qld + 8 * b), make_uint2(0u, 0u));
            sfa[r * sld + b] = 0;
        }
        int64_t i = (int64_t)blockIdx.x * g.R + rho;
        if (i >= g.M) continue;
        int64_t r = reverse ? g.M - 1 - i : i;
        int s = 0;
        while (!(r >= seg.row_start[s] && r < seg.row_start[s + 1])) ++s;
        int64_t seg_lo = seg.row_start[s], seg_hi = seg.row_start[s + 1];
        ColParams cp0, cp1;
        if (!PLAIN) {
            load_cols(seg, s, 2 * b, cp0);
            load_cols(seg, s, 2 * b + 1, cp1);
        }
        for (; i < g.M; i += GR) {
            r = reverse ? g.M - 1 - i : i;
            const uint16_t* xp = x + r * g.ldx + 16 * b;
            const uint4 v0 = ld16(xp), v1 = ld16(xp + 8);
            uint32_t y[8];
            if constexpr (PLAIN) {
                y[0] = v0.x; y[1] = v0.y; y[2] = v0.z; y[3] = v0.w;
                y[4] = v1.x; y[5] = v1.y; y[6] = v1.z; y[7] = v1.w;
            } else {
                if (r < seg_lo || r >= seg_hi) {
                    s = 0;
                    while (!(r >= seg.row_start[s] && r < seg.row_start[s + 1])) ++s;
                    seg_lo = seg.row_start[s];
                    seg_hi = seg.row_start[s + 1];
                    load_cols(seg, s, 2 * b, cp0);
                    load_cols(seg, s, 2 * b + 1, cp1);
                }
                modulate8(v0, cp0, y);
                modulate8(v1, cp1, y + 4);
            }
            pack_block16_store(y, s_g, rg, sg_fast, dr, qdata + r * qld, sfa + r * sld, b);
        }
    }
}

// ---------------------------------------------------------------------------
// SwiGLU producer
//
// g is bf16, so bf16(silu(g)) takes at most 65,536 values.  A fill kernel
// evaluates silu_bf16_value for every bf16 bit pattern into g_silu_lut at the
// start of every SwiGLU call (in stream order, so the table is complete before
// the pass that reads it); each producer workgroup copies the 128 KB table
// into LDS and the per-element work becomes one LDS lookup, one binary32
// product with u and one rounding to bf16.  Concurrent calls on other streams
// rewrite the table with the same values.
// ---------------------------------------------------------------------------
__device__ uint16_t g_silu_lut[65536];

__global__ __launch_bounds__(256) void silu_lut_fill_kernel() {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < 65536u) {
        const float sl = silu_bf16_value(__uint_as_float(i << 16));
        g_silu_lut[i] = (uint16_t)(__float_as_uint(sl) >> 16);
    }
}

constexpr int kLutWords = 65536 * 2 / 16;  // uint4 words in the table

__device__ __forceinline__ void lut_to_lds(uint16_t* slut) {
    const uint4* src = reinterpret_cast<const uint4*>(g_silu_lut);
    uint4* dst = reinterpret_cast<uint4*>(slut);
    for (int i = threadIdx.x; i < kLutWords; i += blockDim.x) dst[i] = src[i];
    __syncthreads();
}

// h = bf16(bf16(silu(g)) * u) for two packed bf16 pairs; bf16(silu(g)) from
// the table (the product of two bf16 values is exact in binary32).
__device__ __forceinline__ uint32_t swiglu2_lut(const uint16_t* lut, uint32_t g2, uint32_t u2) {
    const float sa = __uint_as_float((uint32_t)lut[g2 & 0xFFFFu] << 16);
    const float sb = __uint_as_float((uint32_t)lut[g2 >> 16] << 16);
    return pack_bf16x2(sa * bf16_lo(u2), sb * bf16_hi(u2));
}

__device__ __forceinline__ void swiglu8(const uint16_t* lut, const uint4 gv, const uint4 uv, uint32_t h[4]) {
    h[0] = swiglu2_lut(lut, gv.x, uv.x);
    h[1] = swiglu2_lut(lut, gv.y, uv.y);
    h[2] = swiglu2_lut(lut, gv.z, uv.z);
    h[3] = swiglu2_lut(lut, gv.w, uv.w);
}

__global__ __launch_bounds__(1024) void swiglu_absmax_kernel(const uint16_t* __restrict__ gate,
                                                             const uint16_t* __restrict__ up, RowGeo g,
                                                             uint32_t* ws, float* tensor_scale,
                                                             float* amax_out) {
    __shared__ __attribute__((aligned(16))) uint16_t slut[65536];
    lut_to_lds(slut);
    const int64_t G = gridDim.x;
    uint32_t m2 = 0;
    for (int j = 0; j < g.J; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c >= g.C8) break;
        int64_t r = blockIdx.x;
        for (; r + G < g.M; r += 2 * G) {
            const uint4 g0 = ld16(gate + r * g.ldx + 8 * c), u0 = ld16(up + r * g.ldx + 8 * c);
            const uint4 g1 = ld16(gate + (r + G) * g.ldx + 8 * c), u1 = ld16(up + (r + G) * g.ldx + 8 * c);
            uint32_t h[4];
            swiglu8(slut, g0, u0, h);
#pragma unroll
            for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(h[k]));
            swiglu8(slut, g1, u1, h);
#pragma unroll
            for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(h[k]));
        }
        for (; r < g.M; r += G) {
            uint32_t h[4];
            swiglu8(slut, ld16(gate + r * g.ldx + 8 * c), ld16(up + r * g.ldx + 8 * c), h);
#pragma unroll
            for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(h[k]));
        }
    }
    reduce_and_finish(fold_max(m2), ws, tensor_scale, amax_out);
}


// ---------------------------------------------------------------------------
// Single-pass producer
//
// One launch does both passes.  Every workgroup runs pass 1 over its row
// groups, the workgroups meet at a grid barrier where the global maximum is
// complete, and pass 2 follows in the same launch.  The y values of the row
// groups a workgroup visited last stay on chip across the barrier: the last
// hold_regs() groups in registers, the ones before them in LDS; pass 2 packs
// those first and then reads only the remaining rows from memory again, last
// to first.  The grid never exceeds the workgroups the device holds at once
// (one per CU: the held rows fill the LDS), so the barrier completes on a
// device that other streams do not keep occupied; its wait is bounded in any
// case (see grid_max_barrier).
//
// Thread layout as in the pack passes: thread idx takes block idx % C16 of row
// offset idx / C16 in a group of R rows; workgroup w visits groups w, w+G, ...
// ---------------------------------------------------------------------------
// Row groups held in registers per thread: as many as fit in 128 VGPRs beside
// the working set and the barrier's helper with no spill inside a loop (the
// modulation keeps column parameters live).
constexpr int hold_regs(bool plain) { return plain ? 9 : 7; }
// LDS for held groups (modulation): 32 bytes per active thread and group; at
// D = 5376 (1008 active threads) five groups, with the divisor table and the
// barrier's words beside them within the 160 KB.
constexpr int kModHoldLdsBytes = 158 * 1024;

// Column parameters of one 16-column block as bf16 pairs: bf16(scale+1) and
// shift of columns 2j (low half) and 2j+1 (high half).
struct ColPk {
    uint32_t s1[8];
    uint32_t sh[8];
};

__device__ __forceinline__ void load_cols_pk(const SegParams& seg, int s, int b, ColPk& cp) {
    const uint16_t* sc = seg.scale + (int64_t)s * seg.ld + 16 * b;
    const uint16_t* sh = seg.shift + (int64_t)s * seg.ld + 16 * b;
    const uint4 c0 = ld16(sc), c1 = ld16(sc + 8), h0 = ld16(sh), h1 = ld16(sh + 8);
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float a = __uint_as_float(cw[j] << 16) + 1.0f;
        const float c = __uint_as_float(cw[j] & 0xFFFF0000u) + 1.0f;
        cp.s1[j] = pack_bf16x2(a, c);
        cp.sh[j] = hw[j];
    }
}

// y for 16 consecutive columns: xw = the 8 words of x, y = 8 words of y.
__device__ __forceinline__ void modulate16_pk(const uint32_t xw[8], const ColPk& cp, uint32_t y[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float pa = round_bf16(bf16_lo(xw[j]) * bf16_lo(cp.s1[j]));
        const float pb = round_bf16(bf16_hi(xw[j]) * bf16_hi(cp.s1[j]));
        y[j] = pack_bf16x2(pa + bf16_lo(cp.sh[j]), pb + bf16_hi(cp.sh[j]));
    }
}

__device__ __forceinline__ void ld32(const uint16_t* p, uint32_t w[8]) {
    const uint4 a = ld16(p), c = ld16(p + 8);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = c.x; w[5] = c.y; w[6] = c.z; w[7] = c.w;
}

__device__ __forceinline__ void max16(uint32_t& m2, const uint32_t y[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) m2 = pk_max_u16(m2, mag2(y[k]));
}

// Segment of row r starting from segment s (rows may move either way).
__device__ __forceinline__ int seg_find(const SegParams& seg, int64_t r, int s) {
    while (r >= seg.row_start[s + 1]) ++s;
    while (r < seg.row_start[s]) --s;
    return s;
}

// Workgroup maximum, then the grid barrier of the single launch.
//
// Workspace layout: 32-bit words 0 and 1 belong to the two-pass absmax
// kernels; the single launch uses a result word (64-bit, byte 128), one
// arrival word per workgroup (64-bit, from byte 256) and one claim word per
// workgroup (after the arrival words).  These carry a 44-bit tag above a
// 20-bit payload, and every launch gets a fresh tag from the host, so words
// of earlier launches never match and nothing is ever reset.
//  - arrival: each workgroup stores (tag, its maximum) into its own word, so
//    no two workgroups contend for one word (same-address atomics serialize
//    at ~0.1 us each, which made a counter-based barrier cost 20 us);
//  - workgroup 0 polls every arrival word until all carry the tag, forms the
//    maximum and publishes (tag, published, bits) into the result word with a
//    compare-and-swap; the other workgroups poll the result word;
//  - helping: the barrier needs every workgroup's pass 1, not every
//    workgroup's presence.  A workgroup that has waited `help_ticks` (the CUs
//    it waits for may be held by another launch that waits in turn) scans
//    the arrival words like workgroup 0, claims a workgroup that has not
//    arrived (compare-and-swap on its claim word) and computes that
//    workgroup's pass-1 maximum itself, storing it as its arrival.  The
//    workgroups that could not run find the result published when they do,
//    and go on to their pass 2;
//  - bound: a wait past `wait_ticks` (0: at once) abandons the barrier, also
//    by compare-and-swap on the result word, so exactly one outcome is
//    visible to every workgroup: the true maximum, or NaN.
// Every workgroup that settles the result word writes the tensor scale of
// the outcome that holds (the same value for all of them).
// The LDS flags thread 0 sets (s_done, s_scan, s_help) are read by every wave
// between the workgroup barrier after the write and the one before the next
// write, so all waves take the same branch and meet the same barriers.
constexpr int kResultQword = 16;                        // 64-bit word index (byte 128)
constexpr int kTimeoutCountWord = NVFP4_WORKSPACE_TIMEOUT_COUNT_OFFSET / 4;  // 32-bit word (byte 192)
static_assert(NVFP4_WORKSPACE_TIMEOUT_COUNT_OFFSET % 4 == 0 && NVFP4_WORKSPACE_TIMEOUT_COUNT_OFFSET >= 136 &&
                  NVFP4_WORKSPACE_TIMEOUT_COUNT_OFFSET + 4 <= 256,
              "the count lies in the header, clear of the maximum, counter and result words");
constexpr int kSlotQword = 32;                          // workgroup 0's arrival word (byte 256)
constexpr int kClaimQword = kSlotQword + kMaxGridSlots;  // workgroup 0's claim word
constexpr uint32_t kPublished = 0x10000u, kAbandoned = 0x20000u;
constexpr uint32_t kNanBits = 0x7FC0u;
static_assert(kClaimQword * 8 + 8 * kMaxGridSlots == kWorkspaceBytes, "workspace layout");

__device__ __forceinline__ uint64_t load_dev64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t cas_dev64(uint64_t* p, uint64_t expect, uint64_t v) {
    __hip_atomic_compare_exchange_strong(p, &expect, v, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return expect;  // the value found
}
__device__ __forceinline__ uint64_t tag_of(uint64_t w) { return w >> 20; }
__device__ __forceinline__ uint64_t tagged(uint64_t tag, uint32_t v) { return (tag << 20) | v; }

__device__ __forceinline__ void write_scale(uint32_t bits, float* tensor_scale, float* amax_out) {
    const float amax = __uint_as_float(bits << 16);
    tensor_scale[0] = (amax == 0.0f) ? 1.0f : amax / 2688.0f;
    if (amax_out) amax_out[0] = amax;
}

// Result word -> magnitude bits (NaN for an abandoned barrier).
__device__ __forceinline__ uint32_t outcome_bits(uint64_t r) {
    return ((uint32_t)r & kAbandoned) ? kNanBits : ((uint32_t)r & 0xFFFFu);
}

// Settles the result word of tag `tag`: installs `want` unless a word of this
// tag is already there; returns the word that holds, and in `installed`
// whether this call put it there (one call per launch does).
__device__ __forceinline__ uint64_t settle(uint64_t* res, uint64_t tag, uint64_t want, bool& installed) {
    installed = false;
    uint64_t cur = load_dev64(res);
    while (tag_of(cur) != tag) {
        const uint64_t found = cas_dev64(res, cur, want);
        if (found == cur) {
            installed = true;
            return want;
        }
        cur = found;
    }
    return cur;
}

// Maximum of one value per thread over the workgroup (all threads get it).
__device__ __forceinline__ uint32_t workgroup_max(uint32_t v, uint32_t* red) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nwv = (blockDim.x + 63) >> 6;
    v = wave_max_u32(v);
    __syncthreads();
    if (lane == 0) red[wv] = v;
    __syncthreads();
    uint32_t mm = 0;
    for (int i = 0; i < nwv; ++i) mm = red[i] > mm ? red[i] : mm;
    return mm;
}

// The barrier.  m16: this thread's part of the workgroup's pass-1 maximum
// (bf16 magnitude bits).  help(w) returns this thread's part of workgroup w's
// pass-1 maximum, computed by the calling workgroup (all its threads call it).
template <typename HELP>
__device__ uint32_t grid_max_barrier(uint32_t m16, uint32_t* ws, const BarrierArgs& ba, float* tensor_scale,
                                     float* amax_out, HELP help) {
    __shared__ uint32_t red[16];
    __shared__ uint32_t s_result;
    __shared__ int s_done, s_scan, s_helping, s_cand, s_help;
    __shared__ uint64_t s_t0;
    uint64_t* q = reinterpret_cast<uint64_t*>(ws);
    const int G = (int)gridDim.x;
    const uint64_t tag = ba.tag;
    const int rot0 = (int)blockIdx.x + G / 2;  // helpers start half the grid away from themselves
    const uint32_t mm = workgroup_max(m16, red);
    if (threadIdx.x == 0) {
        store_dev64(&q[kSlotQword + blockIdx.x], tagged(tag, mm));
        s_t0 = __builtin_amdgcn_s_memrealtime();
        s_done = 0;
        s_scan = blockIdx.x == 0;
        s_helping = 0;
    }
    __syncthreads();
    int next = threadIdx.x;  // this thread's first arrival word not yet seen with the tag
    uint32_t mine = 0;       // maximum of the arrival words this thread has seen
    for (;;) {
        // published or abandoned already?
        if (threadIdx.x == 0) {
            const uint64_t r = load_dev64(&q[kResultQword]);
            if (tag_of(r) == tag) {
                s_result = outcome_bits(r);
                s_done = 1;
            }
        }
        __syncthreads();
        if (s_done) break;
        // workgroup 0 and helpers: have all arrived?
        if (s_scan) {
            while (next < G) {
                const uint64_t v = load_dev64(&q[kSlotQword + next]);
                if (tag_of(v) != tag) break;
                mine = ((uint32_t)v & 0xFFFFu) > mine ? ((uint32_t)v & 0xFFFFu) : mine;
                next += blockDim.x;
            }
            if (__syncthreads_and(next >= G)) {
                const uint32_t all = workgroup_max(mine, red);
                if (threadIdx.x == 0) {
                    bool installed;
                    const uint64_t r = settle(&q[kResultQword], tag, tagged(tag, kPublished | all), installed);
                    write_scale(outcome_bits(r), tensor_scale, amax_out);
                    s_result = outcome_bits(r);
                }
                break;
            }
        }
        __syncthreads();  // s_done and s_scan read by every wave
        // the bound; from help_ticks on, help a workgroup that has not arrived
        if (threadIdx.x == 0) {
            const uint64_t el = __builtin_amdgcn_s_memrealtime() - s_t0;
            s_help = -1;
            s_cand = G;
            if (ba.wait_ticks == 0 || el > ba.wait_ticks) {
                bool installed;
                const uint64_t r = settle(&q[kResultQword], tag, tagged(tag, kAbandoned), installed);
                // the one workgroup that abandoned this launch's barrier counts it
                if (installed)
                    __hip_atomic_fetch_add(ws + kTimeoutCountWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                write_scale(outcome_bits(r), tensor_scale, amax_out);
                s_result = outcome_bits(r);
                s_done = 1;
            } else if (el >= ba.help_ticks) {
                s_scan = 1;
                s_helping = 1;
            }
        }
        __syncthreads();
        if (s_done) break;
        if (s_helping) {
            // every thread offers the first arrival word it has not seen with
            // the tag, if that workgroup is still absent and unclaimed; the
            // offer first in rotation order from rot0 is claimed
            if (next < G && tag_of(load_dev64(&q[kSlotQword + next])) != tag &&
                tag_of(load_dev64(&q[kClaimQword + next])) != tag)
                atomicMin(&s_cand, (next - rot0 + 2 * G) % G);
            __syncthreads();
            if (threadIdx.x == 0 && s_cand < G) {
                const int w = (s_cand + rot0) % G;
                const uint64_t c = load_dev64(&q[kClaimQword + w]);
                if (tag_of(c) != tag && cas_dev64(&q[kClaimQword + w], c, tagged(tag, 1u)) == c) s_help = w;
            }
            __syncthreads();
        }
        const int w = s_help;
        if (w >= 0) {
            const uint32_t hm = workgroup_max(help(w), red);
            if (threadIdx.x == 0) store_dev64(&q[kSlotQword + w], tagged(tag, hm));
        } else {
            __builtin_amdgcn_s_sleep(2);
        }
        __syncthreads();  // s_done, s_helping and s_help read by every wave
    }
    __syncthreads();
    return s_result;
}

// Per-workgroup split of its nw row groups: ns streamed (re-read in pass 2),
// nl held in LDS, nr held in registers (the last ones visited).  Only the very
// last group of the tensor can be partial, and it is register-held.
struct HoldSplit {
    int ns, nl, nr;
};
__device__ __forceinline__ HoldSplit hold_split(int64_t groups, int hold_lds, int hold_reg) {
    const int64_t G = gridDim.x, w = blockIdx.x;
    const int nw = w < groups ? (int)((groups - 1 - w) / G + 1) : 0;
    HoldSplit h;
    h.nr = nw < hold_reg ? nw : hold_reg;
    h.nl = (nw - h.nr) < hold_lds ? (nw - h.nr) : hold_lds;
    h.ns = nw - h.nr - h.nl;
    return h;
}

// LDS slot of held group h for thread idx: [h][half][idx] in 16-byte words,
// `active` (the R x blocks-per-row threads that own a block) slots per half,
// so that the idle threads of a workgroup take no LDS.
__device__ __forceinline__ void hold_put(uint4* hold, int active, int h, const uint32_t y[8]) {
    hold[(2 * h) * active + threadIdx.x] = make_uint4(y[0], y[1], y[2], y[3]);
    hold[(2 * h + 1) * active + threadIdx.x] = make_uint4(y[4], y[5], y[6], y[7]);
}
__device__ __forceinline__ void hold_get(const uint4* hold, int active, int h, uint32_t y[8]) {
    const uint4 a = hold[(2 * h) * active + threadIdx.x];
    const uint4 c = hold[(2 * h + 1) * active + threadIdx.x];
    y[0] = a.x; y[1] = a.y; y[2] = a.z; y[3] = a.w;
    y[4] = c.x; y[5] = c.y; y[6] = c.z; y[7] = c.w;
}

__device__ __forceinline__ void zero_pad_rows(const RowGeo& g, uint8_t* qdata, uint8_t* sfa) {
    const int C16 = g.C8 >> 1;
    const int64_t n = (g.rows_total - g.M) * C16;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = g.M + i / C16;
        const int b = (int)(i % C16);
        store_nt(reinterpret_cast<uint2*>(qdata + r * 8 * C16 + 8 * b), make_uint2(0u, 0u));
        sfa[r * C16 + b] = 0;
    }
}

// Modulation of two packed columns with the product rounded by round_bf16
// (one instruction fewer per pair than modulate2; same values).
__device__ __forceinline__ uint32_t modulate2r(uint32_t x2, float s1a, float s1b, float sha, float shb) {
    const float pa = round_bf16(bf16_lo(x2) * s1a), pb = round_bf16(bf16_hi(x2) * s1b);
    return pack_bf16x2(pa + sha, pb + shb);
}

__device__ __forceinline__ void mod16_packed(const uint4& a, const uint4& c, const ColParams& p0, const ColParams& p1,
                                             uint32_t y[8]) {
    const uint32_t xw[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        y[j] = modulate2r(xw[j], p0.s1[2 * j], p0.s1[2 * j + 1], p0.sh[2 * j], p0.sh[2 * j + 1]);
        y[4 + j] = modulate2r(xw[4 + j], p1.s1[2 * j], p1.s1[2 * j + 1], p1.sh[2 * j], p1.sh[2 * j + 1]);
    }
}

// Running maximum of |a| and |b| that propagates NaN (v_maximum3_f32 with
// absolute-value operands).
__device__ __forceinline__ float max_abs2(float m, float a, float b) {
    return __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(__builtin_fabsf(a), __builtin_fabsf(b)));
}

// Largest |s[k]| of 16 values (NaN if any is NaN) as a tree of three-input
// maxima: 8 v_maximum3_f32 (a running maximum pairs values into 12).
__device__ __forceinline__ float absmax16(const float s[16]) {
    auto mx3 = [](float a, float b, float c) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
    };
    float m[6];
#pragma unroll
    for (int i = 0; i < 5; ++i)
        m[i] = mx3(__builtin_fabsf(s[3 * i]), __builtin_fabsf(s[3 * i + 1]), __builtin_fabsf(s[3 * i + 2]));
    m[5] = __builtin_fabsf(s[15]);
    return __builtin_elementwise_maximum(mx3(m[0], m[1], m[2]), mx3(m[3], m[4], m[5]));
}

// Running maximum of the magnitudes of the unrounded modulation sums of 16
// columns (NaN once any sum is NaN).  bf16 rounding is monotone and odd, so
// the bf16 rounding of this maximum is the largest |y| of those columns: pass
// 1 needs no rounded y for rows it does not keep (two VALU operations fewer
// per pair of columns than modulating and taking the maximum of the bits).
__device__ __forceinline__ float mod16_max(const uint4& a, const uint4& c, const ColParams& p0, const ColParams& p1,
                                           float m) {
    const uint32_t xw[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const ColParams& p = j < 4 ? p0 : p1;
        const int k = 2 * (j & 3);
        const float sa = round_bf16(bf16_lo(xw[j]) * p.s1[k]) + p.sh[k];
        const float sb = round_bf16(bf16_hi(xw[j]) * p.s1[k + 1]) + p.sh[k + 1];
        m = max_abs2(m, sa, sb);
    }
    return m;
}

// Largest |bf16(scale+1)| and largest |shift| over a block's 16 columns (NaN if
// any is NaN).
struct ColBound {
    float S, H;
};
__device__ __forceinline__ ColBound col_bound(const ColParams& p0, const ColParams& p1) {
    ColBound cb = {0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        cb.S = __builtin_elementwise_maximum(
            cb.S, __builtin_elementwise_maximum(__builtin_fabsf(p0.s1[k]), __builtin_fabsf(p1.s1[k])));
        cb.H = __builtin_elementwise_maximum(
            cb.H, __builtin_elementwise_maximum(__builtin_fabsf(p0.sh[k]), __builtin_fabsf(p1.sh[k])));
    }
    return cb;
}

// Upper bound on the unrounded modulation sums z = RN32(bf16(x*s1) + sh) of one
// block's 16 columns in two rows of the same segment: with X the largest |x|
// (both rows), |z| <= RN32(bf16(X*S) + H), because |x*s1| <= X*S, bf16 and
// binary32 rounding are monotone and odd, and |p + sh| <= |p| + |sh|.  NaN when
// an x is NaN (its magnitude bits exceed every finite and infinite one).  A
// non-finite bound bounds nothing (x = Inf times s1 = 0 is NaN) and is never
// compared as a bound.
__device__ __forceinline__ float mod_bound2(const uint4& a0, const uint4& a1, const uint4& b0, const uint4& b1,
                                            const ColBound& cb) {
    const uint32_t w[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                            b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    uint32_t m2 = mag2(w[0]);
#pragma unroll
    for (int k = 1; k < 16; ++k) m2 = pk_max_u16(m2, mag2(w[k]));
    const float X = __uint_as_float(fold_max(m2) << 16);
    return round_bf16(X * cb.S) + cb.H;
}

// y of 16 columns as binary32 values (each exactly a bf16) and the largest
// magnitude of the unrounded sums (NaN if any sum is NaN).  Rounding to bf16
// is monotone and odd, so the bf16 rounding of that maximum is the block's
// max |y| (see block_amax_bits).
__device__ __forceinline__ float mod16_f32(const uint4& a, const uint4& c, const ColParams& p0,
                                           const ColParams& p1, float y[16]) {
    const uint32_t xw[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    float z[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const ColParams& p = j < 4 ? p0 : p1;
        const int k = 2 * (j & 3);
        z[2 * j] = round_bf16(bf16_lo(xw[j]) * p.s1[k]) + p.sh[k];
        z[2 * j + 1] = round_bf16(bf16_hi(xw[j]) * p.s1[k + 1]) + p.sh[k + 1];
        y[2 * j] = round_bf16(z[2 * j]);
        y[2 * j + 1] = round_bf16(z[2 * j + 1]);
    }
    return absmax16(z);
}

// bf16 magnitude bits of a block's maximum from the maximum m of its
// unrounded magnitudes: the bf16 rounding of m, or, when m is NaN, the
// largest magnitude bit pattern among the rounded values y (NaN patterns
// rank above Inf and the finite values, as in the global maximum).
__device__ __forceinline__ uint32_t block_amax_bits(float m, const float y[16]) {
    if (m == m) return __float_as_uint(round_bf16(m)) >> 16;
    uint32_t a = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t v = (__float_as_uint(y[k]) >> 16) & 0x7FFFu;
        a = v > a ? v : a;
    }
    return a;
}

// The plain quantizer's y: the input itself, 16 columns as binary32 values,
// and their largest magnitude (NaN if any value is NaN).
__device__ __forceinline__ float plain16_f32(const uint4& a, const uint4& c, float y[16]) {
    const uint32_t xw[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        y[2 * j] = bf16_lo(xw[j]);
        y[2 * j + 1] = bf16_hi(xw[j]);
    }
    return absmax16(y);
}

// Scale and codes of one block given as binary32 values and the maximum from
// mod16_f32.
template <bool BOUNDED = false>
__device__ __forceinline__ PackedBlock pack16f(const float y[16], float m, float s_g, float rg, bool sg_fast,
                                               const float2* dr) {
    const BlockQ bq = block_setup_tab<BOUNDED>(block_amax_bits(m, y), s_g, rg, sg_fast, dr);
    PackedBlock pb;
    pb.w.x = quantize8f(y, bq.d, bq.r, bq.fast) & bq.keep;
    pb.w.y = quantize8f(y + 8, bq.d, bq.r, bq.fast) & bq.keep;
    pb.sf = bq.sf;
    return pb;
}

// h of 16 columns as binary32 values (each exactly a bf16) and the largest
// unrounded magnitude: bf16(silu(g)) from the table times u is exact in
// binary32, and h is its bf16 rounding.
__device__ __forceinline__ float swiglu16_f32(const uint16_t* lut, const uint4& g0, const uint4& g1,
                                              const uint4& u0, const uint4& u1, float h[16]) {
    const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float z[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        z[2 * j] = __uint_as_float((uint32_t)lut[gw[j] & 0xFFFFu] << 16) * bf16_lo(uw[j]);
        z[2 * j + 1] = __uint_as_float((uint32_t)lut[gw[j] >> 16] << 16) * bf16_hi(uw[j]);
        h[2 * j] = round_bf16(z[2 * j]);
        h[2 * j + 1] = round_bf16(z[2 * j + 1]);
    }
    return absmax16(z);
}

// Pass 2 of the SwiGLU producer.  OFF is the offset type: uint32_t when every
// byte offset into gate, up, qdata and sfa fits 32 bits (a uniform base plus
// a 32-bit offset per access), else uint64_t.  One row per iteration: issuing
// two rows' loads at once measured 6% slower.
template <typename OFF>
__global__ __launch_bounds__(1024) void swiglu_pack_kernel(const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ up, RowGeo g,
                                                           const float* tensor_scale,
                                                           uint8_t* __restrict__ qdata,
                                                           uint8_t* __restrict__ sfa, int reverse) {
    __shared__ __attribute__((aligned(16))) uint16_t slut[65536];
    __shared__ float2 dr[128];
    lut_to_lds(slut);
    const float s_g = tensor_scale[0];
    build_dr_table(dr, s_g);
    const bool sg_fast = scale_in_fast_range(s_g);
    const float rg = 1.0f / s_g;
    const char* gb = reinterpret_cast<const char*>(gate);
    const char* ub = reinterpret_cast<const char*>(up);
    const int64_t G = gridDim.x;
    const int C16 = g.C8 >> 1;
    const int64_t qld = 8 * (int64_t)C16, sld = C16;
    const int64_t GR = G * g.R;
    const OFF xrow = (OFF)2 * (OFF)g.ldx;
    for (int j = 0; j < g.J; ++j) {
        const int idx = threadIdx.x + j * blockDim.x;
        const int rho = idx / C16;
        const int b = idx - rho * C16;
        if (rho >= g.R) break;
        for (int64_t r = g.M + (int64_t)blockIdx.x * g.R + rho; r < g.rows_total; r += GR) {
            store_nt(reinterpret_cast<uint2*>(qdata + r * qld + 8 * b), make_uint2(0u, 0u));
            sfa[r * sld + b] = 0;
        }
        const OFF xcol = (OFF)32 * (OFF)b, qcol = (OFF)8 * (OFF)b;
        // Loads after the previous row's stores: issuing them ahead of the
        // stores, as the single launch does, measured 1.7% slower here.
        for (int64_t i = (int64_t)blockIdx.x * g.R + rho; i < g.M; i += GR) {
            const OFF r = (OFF)(reverse ? g.M - 1 - i : i);
            const OFF o = r * xrow + xcol;
            const uint4 g0 = *reinterpret_cast<const uint4*>(gb + o);
            const uint4 g1 = *reinterpret_cast<const uint4*>(gb + o + 16);
            const uint4 u0 = *reinterpret_cast<const uint4*>(ub + o);
            const uint4 u1 = *reinterpret_cast<const uint4*>(ub + o + 16);
            float h[16];
            const float m = swiglu16_f32(slut, g0, g1, u0, u1, h);
            store_block(pack16f(h, m, s_g, rg, sg_fast, dr), qdata + (r * (OFF)qld + qcol),
                        sfa + (r * (OFF)sld + (OFF)b));
        }
    }
}

// Byte offsets within x, qdata and sfa fit 32 bits (checked by the caller),
// so every access is a uniform base pointer plus a 32-bit offset.
__device__ __forceinline__ uint4 ld16o(const char* base, uint32_t off) {
    return *reinterpret_cast<const uint4*>(base + off);
}

// The streamed loops of the modulation single launch as raw buffer accesses:
// a fixed per-lane offset (the lane's row in local group 0 and its column)
// plus a wave-uniform scalar offset (local group t times the grid stride in
// bytes), so that stepping from one row group to the next takes no VALU
// address arithmetic (a 64-bit multiply-add per access before; measured 1-2%
// faster per launch).  In the SwiGLU single launch the same change measured
// slower in pass 2 and no different in pass 1, and it keeps its pointer
// accesses.  Every offset the kernel forms is
// below 2^32 (checked by the caller), within the descriptors' range of
// 2^32 - 1 bytes.
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc32(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0xFFFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// A block's QDATA non-temporally (whole lines per wave) and its scale byte
// plainly, as store_block.
__device__ __forceinline__ void bstore_block(const PackedBlock& pb, __amdgpu_buffer_rsrc_t qr, uint32_t qo,
                                             __amdgpu_buffer_rsrc_t sr, uint32_t so, uint32_t qs, uint32_t ss) {
    __builtin_amdgcn_raw_buffer_store_b64((u32x2v){pb.w.x, pb.w.y}, qr, (int)qo, (int)qs, 2);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)pb.sf, sr, (int)so, (int)ss, 0);
}

// Pass 2 of the single launch: register-held groups, then LDS-held ones,
// then the streamed groups last to first.  Every thread of the workgroup runs
// the loops (`on` guards the memory accesses) so that the streamed loop can
// end each iteration with a workgroup barrier: left to themselves the waves
// of a workgroup drift apart by ~30 us over this loop and the last ones then
// finish alone with too few loads in flight.
template <bool PLAIN, int HR = hold_regs(PLAIN)>
__device__ __forceinline__ void pass2_mod(const char* __restrict__ xb, const RowGeo& g, const SegParams& seg,
                                          const uint32_t (&hy)[HR][8], const uint4* hold, const HoldSplit& hs,
                                          const float2* dr, float s_g, float rg, bool sg_fast, bool on, int r_first,
                                          int gstride, int b, uint8_t* __restrict__ qdata,
                                          uint8_t* __restrict__ sfa) {
    const int C16 = g.C8 >> 1;
    const uint32_t xrow = 2u * (uint32_t)g.ldx, qrow = 8u * (uint32_t)C16, srow = (uint32_t)C16;
    const uint32_t xcol = 32u * (uint32_t)b, qcol = 8u * (uint32_t)b;
    const int t0 = hs.ns + hs.nl;
    if (on) {
#pragma unroll
        for (int h = 0; h < HR; ++h) {
            const int r = r_first + (t0 + h) * gstride;
            if (h < hs.nr && r < g.M)
                pack_block16_store<true>(hy[h], s_g, rg, sg_fast, dr, qdata + (uint32_t)r * qrow, sfa + (uint32_t)r * srow,
                                   b);
        }
        for (int h = hs.nl - 1; h >= 0; --h) {
            const int r = r_first + (hs.ns + h) * gstride;
            uint32_t y[8];
            hold_get(hold, g.R * (g.C8 >> 1), h, y);
            pack_block16_store<true>(y, s_g, rg, sg_fast, dr, qdata + (uint32_t)r * qrow, sfa + (uint32_t)r * srow, b);
        }
    }
    int t = hs.ns - 1;
    if (t < 0) return;  // uniform over the workgroup
    int s2 = 0;
    ColParams c0, c1;  // binary32 parameters: this loop is short of VALU, not of registers
    int seg_lo = 0;    // rows decrease in this loop
    if (!PLAIN && on) {
        s2 = seg_find(seg, r_first + t * gstride, 0);
        load_cols(seg, s2, 2 * b, c0);
        load_cols(seg, s2, 2 * b + 1, c1);
        seg_lo = (int)seg.row_start[s2];
    }
    auto pack = [&](const uint4& v0, const uint4& v1, int r) {
        float y[16];
        float m;
        if constexpr (PLAIN) {
            m = plain16_f32(v0, v1, y);
        } else {
            if (r < seg_lo) {
                s2 = seg_find(seg, r, s2);
                seg_lo = (int)seg.row_start[s2];
                load_cols(seg, s2, 2 * b, c0);
                load_cols(seg, s2, 2 * b + 1, c1);
            }
            m = mod16_f32(v0, v1, c0, c1, y);
        }
        return pack16f<true>(y, m, s_g, rg, sg_fast, dr);
    };
    const __amdgpu_buffer_rsrc_t qr = rsrc32(qdata), sr = rsrc32(sfa);
    const uint32_t qo = (uint32_t)r_first * qrow + qcol, so = (uint32_t)r_first * srow + (uint32_t)b;
    const uint32_t gq = (uint32_t)gstride * qrow, gs = (uint32_t)gstride * srow;
    // local group tt's QDATA and SFA
    auto put = [&](const PackedBlock& pb, int tt) {
        bstore_block(pb, qr, qo, sr, so, (uint32_t)tt * gq, (uint32_t)tt * gs);
    };
    // Two groups per iteration.  Loads and stores share one in-order counter,
    // so a load issued after a store cannot be waited for without waiting for
    // the store too; the next pair's loads are therefore issued before this
    // pair's stores, and the barrier is a bare s_barrier that keeps the waves
    // in step without a memory fence.  With the barrier every wave would
    // otherwise wait out the store latency each iteration (measured 5% slower
    // over the launch; the pack passes without a barrier gain nothing).
    uint4 a0, a1, b0, b1;
    const __amdgpu_buffer_rsrc_t xr = rsrc32(xb);
    const uint32_t xo = (uint32_t)r_first * xrow + xcol, gx = (uint32_t)gstride * xrow;
    auto load_pair = [&](int tt) {
        const uint32_t s0 = (uint32_t)tt * gx, s1 = s0 - gx;
        a0 = bld16(xr, xo, s0);
        a1 = bld16(xr, xo + 16, s0);
        b0 = bld16(xr, xo, s1);
        b1 = bld16(xr, xo + 16, s1);
    };
    if (t >= 1 && on) load_pair(t);
    for (; t >= 1; t -= 2) {
        if (on) {
            const int r0 = r_first + t * gstride, r1 = r0 - gstride;
            const PackedBlock p0 = pack(a0, a1, r0);
            const PackedBlock p1 = pack(b0, b1, r1);
            if (t >= 3) load_pair(t - 2);
            put(p0, t);
            put(p1, t - 1);
        }
        __builtin_amdgcn_s_barrier();
    }
    if (t == 0 && on) put(pack(bld16(xr, xo, 0), bld16(xr, xo + 16, 0), r_first), 0);
}

// PLAIN: the plain quantizer (y = x, no modulation; seg is not read).
template <bool PLAIN>
__global__ __launch_bounds__(1024) void modulate_quantize_kernel(const uint16_t* __restrict__ x, RowGeo g,
                                                                 SegParams seg, uint32_t* ws, float* tensor_scale,
                                                                 float* amax_out, uint8_t* __restrict__ qdata,
                                                                 uint8_t* __restrict__ sfa, int hold_lds,
                                                                 BarrierArgs ba) {
    __shared__ uint4 hold[kModHoldLdsBytes / 16];
    __shared__ float2 dr[128];
    __shared__ uint32_t thr_word;  // pass 1: a maximum counted by a thread of the workgroup
    const char* xb = reinterpret_cast<const char*>(x);
    const int C16 = g.C8 >> 1;
    const int rho = threadIdx.x / C16, b = threadIdx.x - rho * C16;
    const bool on = rho < g.R;
    const int64_t groups = (g.M + g.R - 1) / g.R;
    constexpr int HR = hold_regs(PLAIN);
    const HoldSplit hs = hold_split(groups, hold_lds, HR);
    const int gstride = (int)gridDim.x * g.R;
    const int r_first = (int)blockIdx.x * g.R + rho;  // row of local group 0
    const uint32_t xrow = 2u * (uint32_t)g.ldx, xcol = 32u * (uint32_t)b;

    // ---- pass 1 (every thread runs the loops; `on` guards memory accesses) ----
    if (threadIdx.x == 0) thr_word = 0;
    __syncthreads();
    uint32_t m2 = 0;
    uint32_t hy[HR][8];
    int s = 0, seg_hi = 0;
    ColPk cp;
    if (on) {
        // LDS-held groups first, so that more of the rows read last (before
        // the register-held ones) are rows pass 2 reads again, still in the
        // memory-side cache when it starts (measured 0-2% faster)
        for (int tl = hs.ns; tl < hs.ns + hs.nl; ++tl) {
            const int r = r_first + tl * gstride;
            const uint32_t o = (uint32_t)r * xrow + xcol;
            const uint4 a = ld16o(xb, o), c = ld16o(xb, o + 16);
            const uint32_t v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            uint32_t y[8];
            if constexpr (PLAIN) {
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = v[k];
            } else {
                if (r >= seg_hi) {
                    s = seg_find(seg, r, s);
                    seg_hi = (int)seg.row_start[s + 1];
                    load_cols_pk(seg, s, b, cp);
                }
                modulate16_pk(v, cp, y);
            }
            max16(m2, y);
            hold_put(hold, g.R * C16, tl - hs.ns, y);
        }
    }
    // streamed groups, two per iteration, with binary32 column parameters
    // (short of VALU here, not of registers: the held groups come later).
    // EXACT: the maximum of the rounded y's bit patterns (the plain quantizer,
    // and the rare rerun after a NaN); otherwise the maximum of the unrounded
    // sums (mod16_max), whose bf16 rounding is the same value.  Without EXACT a
    // wave skips the modulation of a pair of rows when every thread's bound
    // (mod_bound2) is finite and at most a maximum that a thread of the
    // workgroup has already counted: those sums cannot raise the maximum.
    auto streamed = [&](auto exact) {
        constexpr bool EXACT = decltype(exact)::value;
        constexpr bool BOUND = !PLAIN && !EXACT;
        ColParams c0, c1;
        ColBound cb = {0.0f, 0.0f};
        int hi = 0, sc = 0;
        float mf = 0.0f;
        float thr = 0.0f;  // wave-uniform
        auto cols = [&](int s_) {
            load_cols(seg, s_, 2 * b, c0);
            load_cols(seg, s_, 2 * b + 1, c1);
            if constexpr (BOUND) cb = col_bound(c0, c1);
        };
        if (!PLAIN && on) {
            sc = seg_find(seg, r_first < g.M ? r_first : 0, 0);
            cols(sc);
            hi = (int)seg.row_start[sc + 1];
        }
        auto absmax = [&](const uint4& v0, const uint4& v1, int r) {
            if constexpr (PLAIN) {
                const uint32_t y[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                max16(m2, y);
            } else {
                if (r >= hi) {
                    sc = seg_find(seg, r, sc);
                    hi = (int)seg.row_start[sc + 1];
                    cols(sc);
                }
                if constexpr (EXACT) {
                    uint32_t y[8];
                    mod16_packed(v0, v1, c0, c1, y);
                    max16(m2, y);
                } else {
                    mf = mod16_max(v0, v1, c0, c1, mf);
                }
            }
        };
        const __amdgpu_buffer_rsrc_t xr1 = rsrc32(xb);
        const uint32_t xo1 = (uint32_t)r_first * xrow + xcol, gx1 = (uint32_t)gstride * xrow;
        int t = 0;
        for (; t + 1 < hs.ns; t += 2) {
            const int r0 = r_first + t * gstride, r1 = r0 + gstride;
            uint4 a0, a1, b0, b1;
            bool bounded = true;
            if (on) {
                const uint32_t s0 = (uint32_t)t * gx1, s1 = s0 + gx1;
                a0 = bld16(xr1, xo1, s0);
                a1 = bld16(xr1, xo1 + 16, s0);
                b0 = bld16(xr1, xo1, s1);
                b1 = bld16(xr1, xo1 + 16, s1);
                if constexpr (BOUND) {
                    const float B = mod_bound2(a0, a1, b0, b1, cb);
                    bounded = r1 < hi && B <= thr && B <= 0x1.fffffep127f;
                }
            }
            if constexpr (BOUND) {
                if (!__all(bounded) && on) {
                    absmax(a0, a1, r0);
                    absmax(b0, b1, r1);
                }
                if (((t >> 1) & 3) == 0) thr = raise_threshold(&thr_word, mf);
            } else if (on) {
                absmax(a0, a1, r0);
                absmax(b0, b1, r1);
            }
        }
        if (t < hs.ns && on)
            absmax(bld16(xr1, xo1, (uint32_t)t * gx1), bld16(xr1, xo1 + 16, (uint32_t)t * gx1), r_first + t * gstride);
        return mf;
    };
    if constexpr (PLAIN) {
        streamed(std::true_type{});
    } else {
        const float mf = streamed(std::false_type{});
        if (mf == mf)
            m2 = pk_max_u16(m2, __float_as_uint(round_bf16(mf)) >> 16);
        else
            streamed(std::true_type{});  // a NaN: the largest NaN bit pattern, exactly
    }
    if (on) {
        // register-held groups: all loads first, then y in place of x
        const int t0 = hs.ns + hs.nl;
#pragma unroll
        for (int h = 0; h < HR; ++h) {
            const int r = r_first + (t0 + h) * gstride;
            if (h < hs.nr && r < g.M) {
                const uint32_t o = (uint32_t)r * xrow + xcol;
                const uint4 a = ld16o(xb, o), c = ld16o(xb, o + 16);
                hy[h][0] = a.x; hy[h][1] = a.y; hy[h][2] = a.z; hy[h][3] = a.w;
                hy[h][4] = c.x; hy[h][5] = c.y; hy[h][6] = c.z; hy[h][7] = c.w;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) hy[h][k] = 0u;
            }
        }
#pragma unroll
        for (int h = 0; h < HR; ++h) {
            const int r = r_first + (t0 + h) * gstride;
            const bool valid = h < hs.nr && r < g.M;
            if constexpr (!PLAIN) {
                if (valid && r >= seg_hi) {
                    s = seg_find(seg, r, s);
                    seg_hi = (int)seg.row_start[s + 1];
                    load_cols_pk(seg, s, b, cp);
                }
                uint32_t y[8];
                modulate16_pk(hy[h], cp, y);
#pragma unroll
                for (int k = 0; k < 8; ++k) hy[h][k] = y[k];
            }
            if (valid) max16(m2, hy[h]);
        }
    }
    // pass 1 of workgroup w, for the barrier's helping (see grid_max_barrier);
    // 8 columns at a time and the column parameters loaded per row, so that
    // it needs few registers beside the held rows
    auto help = [=, &seg](int w) -> uint32_t {
        (void)seg;  // read only when modulating
        uint32_t hm2 = 0;
        if (on) {
            const int wf = w * g.R + rho;
            const int nwm = w < groups ? (int)((groups - 1 - w) / gridDim.x + 1) : 0;
            int hs2 = 0;
            for (int t2 = 0; t2 < nwm; ++t2) {
                const int r = wf + t2 * gstride;
                if (r >= g.M) break;
                if constexpr (!PLAIN) hs2 = seg_find(seg, r, hs2);
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint4 a = ld16o(xb, (uint32_t)r * xrow + xcol + 16u * half);
                    uint32_t y[4] = {a.x, a.y, a.z, a.w};
                    if constexpr (!PLAIN) {
                        const uint16_t* sc = seg.scale + (int64_t)hs2 * seg.ld + 16 * b + 8 * half;
                        const uint16_t* sh = seg.shift + (int64_t)hs2 * seg.ld + 16 * b + 8 * half;
                        const uint4 c4 = ld16(sc), h4 = ld16(sh);
                        const uint32_t cw[4] = {c4.x, c4.y, c4.z, c4.w};
                        const uint32_t hw[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            y[j] = modulate2r(y[j], mod_scale1((uint16_t)(cw[j] & 0xFFFFu)),
                                              mod_scale1((uint16_t)(cw[j] >> 16)), bf16_lo(hw[j]), bf16_hi(hw[j]));
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) hm2 = pk_max_u16(hm2, mag2(y[j]));
                }
            }
        }
        return fold_max(hm2);
    };
    const uint32_t bits = grid_max_barrier(fold_max(m2), ws, ba, tensor_scale, amax_out, help);

    // ---- pass 2 ----
    const float amax = __uint_as_float(bits << 16);
    const float s_g = (amax == 0.0f) ? 1.0f : amax / 2688.0f;
    build_dr_table(dr, s_g);
    const bool sg_fast = scale_in_fast_range(s_g);
    const float rg = 1.0f / s_g;
    zero_pad_rows(g, qdata, sfa);
    pass2_mod<PLAIN>(xb, g, seg, hy, hold, hs, dr, s_g, rg, sg_fast, on, r_first, gstride, b, qdata, sfa);
}

// ---------------------------------------------------------------------------
// Single-launch SwiGLU producer
//
// The structure of the modulation single launch with the SwiGLU input: h of
// the row groups a workgroup visits last stays in registers across the grid
// barrier (the silu table fills the LDS, so none is held there); pass 2 packs
// those first and reads gate and up again for the rest, last to first.  The
// silu table is filled by silu_lut_fill_kernel before the launch.
// ---------------------------------------------------------------------------
constexpr int kSwigluHoldRegs = 9;  // row groups held in registers per thread (as hold_regs)

// h of 16 columns as packed bf16 words (the pass-1 form, also what is held).
__device__ __forceinline__ void swiglu16_pk(const uint16_t* lut, const uint4& g0, const uint4& g1, const uint4& u0,
                                            const uint4& u1, uint32_t h[8]) {
    swiglu8(lut, g0, u0, h);
    swiglu8(lut, g1, u1, h + 4);
}

__global__ __launch_bounds__(1024) void swiglu_quantize_kernel(const uint16_t* __restrict__ gate,
                                                               const uint16_t* __restrict__ up, RowGeo g,
                                                               uint32_t* ws, float* tensor_scale, float* amax_out,
                                                               uint8_t* __restrict__ qdata,
                                                               uint8_t* __restrict__ sfa, BarrierArgs ba) {
    __shared__ __attribute__((aligned(16))) uint16_t slut[65536];
    __shared__ float2 dr[128];
    lut_to_lds(slut);
    const char* gb = reinterpret_cast<const char*>(gate);
    const char* ub = reinterpret_cast<const char*>(up);
    const int C16 = g.C8 >> 1;
    const int rho = threadIdx.x / C16, b = threadIdx.x - rho * C16;
    const bool on = rho < g.R;
    const int64_t groups = (g.M + g.R - 1) / g.R;
    constexpr int HR = kSwigluHoldRegs;
    const HoldSplit hs = hold_split(groups, 0, HR);
    const int gstride = (int)gridDim.x * g.R;
    const int r_first = (int)blockIdx.x * g.R + rho;  // row of local group 0
    const uint32_t xrow = 2u * (uint32_t)g.ldx, xcol = 32u * (uint32_t)b;

    // ---- pass 1: every streamed group for its maximum, then the held ones ----
    uint32_t m2 = 0;
    uint32_t hy[HR][8];
    if (on) {
        for (int t = 0; t < hs.ns; ++t) {
            const uint32_t o = (uint32_t)(r_first + t * gstride) * xrow + xcol;
            uint32_t h[8];
            swiglu16_pk(slut, ld16o(gb, o), ld16o(gb, o + 16), ld16o(ub, o), ld16o(ub, o + 16), h);
            max16(m2, h);
        }
#pragma unroll
        for (int k = 0; k < HR; ++k) {
            const int r = r_first + (hs.ns + k) * gstride;
            if (k < hs.nr && r < g.M) {
                const uint32_t o = (uint32_t)r * xrow + xcol;
                swiglu16_pk(slut, ld16o(gb, o), ld16o(gb, o + 16), ld16o(ub, o), ld16o(ub, o + 16), hy[k]);
                max16(m2, hy[k]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) hy[k][j] = 0u;
            }
        }
    }
    // pass 1 of workgroup w, for the barrier's helping (see grid_max_barrier)
    auto help = [=](int w) -> uint32_t {
        uint32_t hm2 = 0;
        if (on) {
            const int wf = w * g.R + rho;
            const int nwm = w < groups ? (int)((groups - 1 - w) / gridDim.x + 1) : 0;
            for (int t2 = 0; t2 < nwm; ++t2) {
                const int r = wf + t2 * gstride;
                if (r >= g.M) break;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t o = (uint32_t)r * xrow + xcol + 16u * half;
                    uint32_t h[4];
                    swiglu8(slut, ld16o(gb, o), ld16o(ub, o), h);
#pragma unroll
                    for (int j = 0; j < 4; ++j) hm2 = pk_max_u16(hm2, mag2(h[j]));
                }
            }
        }
        return fold_max(hm2);
    };
    const uint32_t bits = grid_max_barrier(fold_max(m2), ws, ba, tensor_scale, amax_out, help);

    // ---- pass 2 ----
    const float amax = __uint_as_float(bits << 16);
    const float s_g = (amax == 0.0f) ? 1.0f : amax / 2688.0f;
    build_dr_table(dr, s_g);
    const bool sg_fast = scale_in_fast_range(s_g);
    const float rg = 1.0f / s_g;
    zero_pad_rows(g, qdata, sfa);
    const uint32_t qrow = 8u * (uint32_t)C16, srow = (uint32_t)C16;
    const uint32_t qcol = 8u * (uint32_t)b;
    if (on) {
#pragma unroll
        for (int k = 0; k < HR; ++k) {
            const int r = r_first + (hs.ns + k) * gstride;
            if (k < hs.nr && r < g.M)
                pack_block16_store<true>(hy[k], s_g, rg, sg_fast, dr, qdata + (uint32_t)r * qrow, sfa + (uint32_t)r * srow,
                                   b);
        }
    }
    auto put = [&](const PackedBlock& pb, int r) {
        store_block(pb, qdata + ((uint32_t)r * qrow + qcol), sfa + ((uint32_t)r * srow + b));
    };
    auto pack = [&](const uint4& g0, const uint4& g1, const uint4& u0, const uint4& u1) {
        float h[16];
        const float m = swiglu16_f32(slut, g0, g1, u0, u1, h);
        return pack16f<true>(h, m, s_g, rg, sg_fast, dr);
    };
    // Streamed groups last to first, two per iteration, as in the modulation
    // single launch: the next pair's loads ahead of this pair's stores, and a
    // bare s_barrier keeping the waves in step.
    int t = hs.ns - 1;
    if (t < 0) return;  // uniform over the workgroup
    uint4 ga0, ga1, ua0, ua1, gb0, gb1, ub0, ub1;
    auto load_pair = [&](int tt) {
        const uint32_t o0 = (uint32_t)(r_first + tt * gstride) * xrow + xcol;
        const uint32_t o1 = o0 - (uint32_t)gstride * xrow;
        ga0 = ld16o(gb, o0);
        ga1 = ld16o(gb, o0 + 16);
        ua0 = ld16o(ub, o0);
        ua1 = ld16o(ub, o0 + 16);
        gb0 = ld16o(gb, o1);
        gb1 = ld16o(gb, o1 + 16);
        ub0 = ld16o(ub, o1);
        ub1 = ld16o(ub, o1 + 16);
    };
    if (t >= 1 && on) load_pair(t);
    for (; t >= 1; t -= 2) {
        if (on) {
            const int r0 = r_first + t * gstride, r1 = r0 - gstride;
            const PackedBlock p0 = pack(ga0, ga1, ua0, ua1);
            const PackedBlock p1 = pack(gb0, gb1, ub0, ub1);
            if (t >= 3) load_pair(t - 2);
            put(p0, r0);
            put(p1, r1);
        }
        __builtin_amdgcn_s_barrier();
    }
    if (t == 0 && on) {
        const uint32_t o0 = (uint32_t)r_first * xrow + xcol;
        put(pack(ld16o(gb, o0), ld16o(gb, o0 + 16), ld16o(ub, o0), ld16o(ub, o0 + 16)), r_first);
    }
}

// ---------------------------------------------------------------------------
// Single-step kernels (elementwise, grid-stride)
// ---------------------------------------------------------------------------
__global__ void step_modulate_kernel(const uint16_t* x, const uint16_t* sc, const uint16_t* sh, uint16_t* y,
                                     int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const float s1 = mod_scale1(sc[i]);
        const float h = __uint_as_float((uint32_t)sh[i] << 16);
        y[i] = (uint16_t)(modulate2((uint32_t)x[i], s1, s1, h, h) & 0xFFFF);
    }
}

// Reads the same table as the producer (from global memory), so that checking
// this step over all inputs checks every table entry the producer can use.
__global__ void step_swiglu_kernel(const uint16_t* g, const uint16_t* u, uint16_t* h, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        h[i] = (uint16_t)(swiglu2_lut(g_silu_lut, (uint32_t)g[i], (uint32_t)u[i]) & 0xFFFF);
}

__global__ void step_block_scale_kernel(const uint16_t* a16, const float* sgp, uint8_t* sf, int64_t n) {
    const float s_g = sgp[0];
    const bool sg_fast = scale_in_fast_range(s_g);
    const float rg = 1.0f / s_g;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const BlockQ b = block_setup((uint32_t)(a16[i] & 0x7FFF), s_g, rg, sg_fast);
        sf[i] = (uint8_t)b.sf;
    }
}

// Element code of y[i] given the block scale sf[i].  In a tensor every value
// of a block satisfies |y| <= 9*d (d = sf*s_g, the block scale having been
// derived from the block maximum), and the producer takes the Markstein
// quotient there whenever s_g is in the fast range and the block maximum is
// finite.  Pairs (y, sf) outside that relation cannot occur in a tensor; for
// them the correctly rounded division is used.
__global__ void step_element_code_kernel(const uint16_t* y, const uint8_t* sfp, const float* sgp, uint8_t* code,
                                         int64_t n) {
    const float s_g = sgp[0];
    const bool sg_fast = scale_in_fast_range(s_g);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t sf = sfp[i];
        const float d = e4m3_value(sf) * s_g;
        const float r = 1.0f / d;
        const float ya = __uint_as_float((uint32_t)(y[i] & 0x7FFF) << 16);
        const bool fast = sg_fast && ((y[i] & 0x7FFF) < 0x7F80) && ya <= 16.0f * d;
        const uint32_t keep = (sf == 0u || sf == 0x7Fu) ? 0u : 0xFu;
        uint32_t yy[4] = {(uint32_t)y[i], 0u, 0u, 0u};
        const uint32_t w = quantize8(yy, d, r, fast);
        code[i] = (uint8_t)(w & keep);
    }
}

__global__ void step_e2m1_kernel(const float* v, uint8_t* code, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        code[i] = (uint8_t)(fp4_pack2<0>(0u, v[i], 0.0f) & 0xF);
}

__global__ void step_e4m3_kernel(const float* t, uint8_t* code, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        code[i] = (uint8_t)e4m3_encode(t[i]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int step_grid(int64_t n) {
    int64_t b = (n + 255) / 256;
    return (int)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

hipError_t launch_modulate_absmax(const uint16_t* x, const RowGeo& g, const SegParams& seg, uint32_t* ws,
                                  float* tensor_scale, float* amax_out, bool plain, hipStream_t s) {
    if (plain)
        hipLaunchKernelGGL(modulate_absmax_kernel<true>, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, ws, tensor_scale,
                           amax_out);
    else
        hipLaunchKernelGGL(modulate_absmax_kernel<false>, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, ws,
                           tensor_scale, amax_out);
    return hipGetLastError();
}

hipError_t launch_modulate_pack(const uint16_t* x, const RowGeo& g, const SegParams& seg, const float* tensor_scale,
                                uint8_t* qdata, uint8_t* sfa, bool plain, hipStream_t s) {
    if (plain)
        hipLaunchKernelGGL(modulate_pack_kernel<true>, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, tensor_scale, qdata,
                           sfa, g.reverse);
    else
        hipLaunchKernelGGL(modulate_pack_kernel<false>, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, tensor_scale,
                           qdata, sfa, g.reverse);
    return hipGetLastError();
}

// Workgroups of the single-launch kernel that the current device holds at
// once (occupancy of a 1024-thread workgroup, which bounds every smaller one,
// times the CU count), capped at the workspace's arrival words; cached per
// device.  0 when it cannot be determined.
static int resident_grid(const void* kernel, int* cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    if (cache[dev] >= 0) return cache[dev];
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 1024, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int n = cus * per_cu;
    cache[dev] = n < kMaxGridSlots ? n : kMaxGridSlots;
    return cache[dev];
}

int modulate_quantize_grid() {
    static int cache[kMaxDevices] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1,
                                     -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
    // both instantiations have the same resources (the held rows fill the registers and LDS)
    return resident_grid((const void*)modulate_quantize_kernel<false>, cache);
}

static void launch_silu_fill(hipStream_t s) {
    hipLaunchKernelGGL(silu_lut_fill_kernel, dim3(256), dim3(256), 0, s);
}

int swiglu_quantize_grid() {
    static int cache[kMaxDevices] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1,
                                     -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
    return resident_grid((const void*)swiglu_quantize_kernel, cache);
}

hipError_t launch_swiglu_quantize(const uint16_t* gate, const uint16_t* up, const RowGeo& g, uint32_t* ws,
                                  float* tensor_scale, float* amax_out, uint8_t* qdata, uint8_t* sfa,
                                  const BarrierArgs& ba, hipStream_t s) {
    launch_silu_fill(s);
    hipLaunchKernelGGL(swiglu_quantize_kernel, dim3(g.grid), dim3(g.block), 0, s, gate, up, g, ws, tensor_scale,
                       amax_out, qdata, sfa, ba);
    return hipGetLastError();
}

// A plain launch: the grid never exceeds what the device holds at once, so on
// a device not kept busy by other streams every workgroup is resident and the
// barrier completes (its wait is bounded in any case).  The cooperative launch
// API would guarantee residency but costs tens of microseconds per launch.
hipError_t launch_modulate_quantize(const uint16_t* x, const RowGeo& g, const SegParams& seg, uint32_t* ws,
                                    float* tensor_scale, float* amax_out, uint8_t* qdata, uint8_t* sfa, bool plain,
                                    const BarrierArgs& ba, hipStream_t s) {
    const int hold_lds = kModHoldLdsBytes / (32 * g.R * (g.C8 >> 1));
    if (plain)
        hipLaunchKernelGGL(modulate_quantize_kernel<true>, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, ws,
                           tensor_scale, amax_out, qdata, sfa, hold_lds, ba);
    else
        hipLaunchKernelGGL(modulate_quantize_kernel<false>, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, ws,
                           tensor_scale, amax_out, qdata, sfa, hold_lds, ba);
    return hipGetLastError();
}


hipError_t launch_swiglu_absmax(const uint16_t* gate, const uint16_t* up, const RowGeo& g, uint32_t* ws,
                                float* tensor_scale, float* amax_out, bool fill, hipStream_t s) {
    if (fill) launch_silu_fill(s);
    hipLaunchKernelGGL(swiglu_absmax_kernel, dim3(g.grid), dim3(g.block), 0, s, gate, up, g, ws, tensor_scale,
                       amax_out);
    return hipGetLastError();
}

hipError_t launch_swiglu_pack(const uint16_t* gate, const uint16_t* up, const RowGeo& g, const float* tensor_scale,
                              uint8_t* qdata, uint8_t* sfa, bool fill, hipStream_t s) {
    if (fill) launch_silu_fill(s);
    const bool off32 = ((g.M - 1) * g.ldx + 8 * (int64_t)g.C8) * 2 < ((int64_t)1 << 32) &&
                       g.rows_total * 4 * (int64_t)g.C8 < ((int64_t)1 << 32);
    if (off32)
        hipLaunchKernelGGL(swiglu_pack_kernel<uint32_t>, dim3(g.grid), dim3(g.block), 0, s, gate, up, g, tensor_scale,
                           qdata, sfa, g.reverse);
    else
        hipLaunchKernelGGL(swiglu_pack_kernel<uint64_t>, dim3(g.grid), dim3(g.block), 0, s, gate, up, g, tensor_scale,
                           qdata, sfa, g.reverse);
    return hipGetLastError();
}

// Zeroes a workspace of `bytes` (a multiple of 16) with vector stores, in
// stream order: a kernel rather than a memset, so that a call captured into a
// graph clears the words again on every replay.
__global__ __launch_bounds__(256) void clear_words_kernel(uint4* __restrict__ p, int n16) {
    for (int i = threadIdx.x; i < n16; i += blockDim.x) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_clear_workspace(void* ws, size_t bytes, hipStream_t s) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, s, (uint4*)ws, (int)(bytes / 16));
    return hipGetLastError();
}

hipError_t launch_step(int which, const void* a, const void* b, const void* c, void* out, int64_t n, hipStream_t s) {
    const dim3 grid(step_grid(n)), block(256);
    switch (which) {
    case STEP_MODULATE:
        hipLaunchKernelGGL(step_modulate_kernel, grid, block, 0, s, (const uint16_t*)a, (const uint16_t*)b,
                           (const uint16_t*)c, (uint16_t*)out, n);
        break;
    case STEP_SWIGLU:
        launch_silu_fill(s);
        hipLaunchKernelGGL(step_swiglu_kernel, grid, block, 0, s, (const uint16_t*)a, (const uint16_t*)b,
                           (uint16_t*)out, n);
        break;
    case STEP_BLOCK_SCALE:
        hipLaunchKernelGGL(step_block_scale_kernel, grid, block, 0, s, (const uint16_t*)a, (const float*)b,
                           (uint8_t*)out, n);
        break;
    case STEP_ELEMENT_CODE:
        hipLaunchKernelGGL(step_element_code_kernel, grid, block, 0, s, (const uint16_t*)a, (const uint8_t*)b,
                           (const float*)c, (uint8_t*)out, n);
        break;
    case STEP_E2M1:
        hipLaunchKernelGGL(step_e2m1_kernel, grid, block, 0, s, (const float*)a, (uint8_t*)out, n);
        break;
    case STEP_E4M3:
        hipLaunchKernelGGL(step_e4m3_kernel, grid, block, 0, s, (const float*)a, (uint8_t*)out, n);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace nvfp4
