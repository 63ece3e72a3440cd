// NVFP4 activation producer kernels for gfx950.
//
// Two passes over the BF16 input, as the exact two-phase design requires
// ("NVFP4 Streaming Design", Numerical Constraint: no tile can be packed
// before the global reduction completes; "NVFP4 Modulation Producer Fusion",
// Dataflow: read the normalized input, reproduce the BF16 modulation and
// reduce |y| without writing y; read it again and write QDATA/SFA into
// caller-owned buffers).
//
// Layout of the work: one thread owns one 8-column chunk (16 bytes of bf16)
// of every row in its workgroup's row range.  A workgroup spans every chunk of
// a row (blockDim = chunks per row rounded up to 64, a thread taking several
// chunks when a row has more than 1024), so each row is read with contiguous
// 16-byte loads and the per-column shift/scale stay in registers for the whole
// row range.  Two neighbouring lanes hold one 16-value block; they exchange
// their partial maxima with one DPP move.
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

// Maximum of the partner lane (lane ^ 1) via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ uint32_t partner_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

// Workgroup maximum of a 16-bit magnitude, then the grid-level finish: one
// atomic max per workgroup; the last workgroup to arrive turns the maximum
// into the tensor scale and returns the workspace to zero.
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
        atomicMax(&ws[0], mm);
        __threadfence();
        const uint32_t ticket = atomicAdd(&ws[1], 1u);
        if (ticket == gridDim.x - 1) {
            __threadfence();
            const uint32_t bits = atomicMax(&ws[0], 0u);
            const float amax = __uint_as_float(bits << 16);
            // s_g = amax / (6 * 448), or 1 when the tensor is all zero
            const float sg = (amax == 0.0f) ? 1.0f : amax / 2688.0f;
            tensor_scale[0] = sg;
            if (amax_out) amax_out[0] = amax;
            atomicExch(&ws[0], 0u);
            atomicExch(&ws[1], 0u);
        }
    }
}

// Per-lane block setup shared by the pack kernels: the block maximum is the
// max of this lane's 8 magnitudes and its partner's.
__device__ __forceinline__ void pack_block_store(const uint32_t y[4], float s_g, float rg, bool sg_fast,
                                                 uint8_t* __restrict__ qrow, uint8_t* __restrict__ srow,
                                                 int c) {
    uint32_t m2 = mag2(y[0]);
    m2 = pk_max_u16(m2, mag2(y[1]));
    m2 = pk_max_u16(m2, mag2(y[2]));
    m2 = pk_max_u16(m2, mag2(y[3]));
    uint32_t m = fold_max(m2);
    const uint32_t p = partner_u32(m);
    m = m > p ? m : p;
    const BlockQ b = block_setup(m, s_g, rg, sg_fast);
    const uint32_t w = quantize8(y, b.d, b.r, b.fast) & b.keep;
    *reinterpret_cast<uint32_t*>(qrow + 4 * c) = w;
    if ((c & 1) == 0) srow[c >> 1] = (uint8_t)b.sf;
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

__global__ __launch_bounds__(1024) void modulate_absmax_kernel(const uint16_t* __restrict__ x, RowGeo g,
                                                               SegParams seg, uint32_t* ws,
                                                               float* tensor_scale, float* amax_out) {
    const int64_t r0 = (int64_t)blockIdx.x * g.rows_per_wg;
    const int64_t r1 = r0 + g.rows_per_wg < g.M ? r0 + g.rows_per_wg : g.M;
    uint32_t m2 = 0;
    for (int j = 0; j < g.J; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c >= g.C8) break;
        for (int s = 0; s < seg.count; ++s) {
            const int64_t a = r0 > seg.row_start[s] ? r0 : seg.row_start[s];
            const int64_t b = r1 < seg.row_start[s + 1] ? r1 : seg.row_start[s + 1];
            if (a >= b) continue;
            ColParams cp;
            load_cols(seg, s, c, cp);
            const uint16_t* xp = x + a * g.ldx + 8 * c;
            int64_t r = a;
            for (; r + 4 <= b; r += 4) {
                uint4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = ld16(xp + u * g.ldx);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    uint32_t y[4];
                    modulate8(v[u], cp, y);
#pragma unroll
                    for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(y[k]));
                }
                xp += 4 * g.ldx;
            }
            for (; r < b; ++r) {
                uint32_t y[4];
                modulate8(ld16(xp), cp, y);
#pragma unroll
                for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(y[k]));
                xp += g.ldx;
            }
        }
    }
    reduce_and_finish(fold_max(m2), ws, tensor_scale, amax_out);
}

__global__ __launch_bounds__(1024) void modulate_pack_kernel(const uint16_t* __restrict__ x, RowGeo g,
                                                             SegParams seg, const float* tensor_scale,
                                                             uint8_t* __restrict__ qdata,
                                                             uint8_t* __restrict__ sfa, int reverse) {
    const float s_g = tensor_scale[0];
    const bool sg_fast = scale_in_fast_range(s_g);
    const float rg = 1.0f / s_g;
    const int64_t tile = reverse ? (int64_t)(gridDim.x - 1 - blockIdx.x) : (int64_t)blockIdx.x;
    const int64_t r0 = tile * g.rows_per_wg;
    const int64_t r1 = r0 + g.rows_per_wg < g.rows_total ? r0 + g.rows_per_wg : g.rows_total;
    const int64_t qld = 4 * (int64_t)g.C8, sld = g.C8 >> 1;
    for (int j = 0; j < g.J; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c >= g.C8) break;
        const int64_t rm = r1 < g.M ? r1 : g.M;
        for (int s = 0; s < seg.count; ++s) {
            const int64_t a = r0 > seg.row_start[s] ? r0 : seg.row_start[s];
            const int64_t b = rm < seg.row_start[s + 1] ? rm : seg.row_start[s + 1];
            if (a >= b) continue;
            ColParams cp;
            load_cols(seg, s, c, cp);
            const uint16_t* xp = x + a * g.ldx + 8 * c;
            int64_t r = a;
            for (; r + 2 <= b; r += 2) {
                const uint4 v0 = ld16(xp), v1 = ld16(xp + g.ldx);
                uint32_t y[4];
                modulate8(v0, cp, y);
                pack_block_store(y, s_g, rg, sg_fast, qdata + r * qld, sfa + r * sld, c);
                modulate8(v1, cp, y);
                pack_block_store(y, s_g, rg, sg_fast, qdata + (r + 1) * qld, sfa + (r + 1) * sld, c);
                xp += 2 * g.ldx;
            }
            for (; r < b; ++r) {
                uint32_t y[4];
                modulate8(ld16(xp), cp, y);
                pack_block_store(y, s_g, rg, sg_fast, qdata + r * qld, sfa + r * sld, c);
                xp += g.ldx;
            }
        }
        // zero padding rows M .. rows_total-1
        for (int64_t r = (r0 > g.M ? r0 : g.M); r < r1; ++r) {
            *reinterpret_cast<uint32_t*>(qdata + r * qld + 4 * c) = 0u;
            if ((c & 1) == 0) sfa[r * sld + (c >> 1)] = 0;
        }
    }
}

// ---------------------------------------------------------------------------
// SwiGLU producer
// ---------------------------------------------------------------------------
__device__ __forceinline__ void swiglu8(const uint4 gv, const uint4 uv, uint32_t h[4]) {
    h[0] = swiglu2(gv.x, uv.x);
    h[1] = swiglu2(gv.y, uv.y);
    h[2] = swiglu2(gv.z, uv.z);
    h[3] = swiglu2(gv.w, uv.w);
}

__global__ __launch_bounds__(1024) void swiglu_absmax_kernel(const uint16_t* __restrict__ gate,
                                                             const uint16_t* __restrict__ up, RowGeo g,
                                                             uint32_t* ws, float* tensor_scale,
                                                             float* amax_out) {
    const int64_t r0 = (int64_t)blockIdx.x * g.rows_per_wg;
    const int64_t r1 = r0 + g.rows_per_wg < g.M ? r0 + g.rows_per_wg : g.M;
    uint32_t m2 = 0;
    for (int j = 0; j < g.J; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c >= g.C8) break;
        const uint16_t* gp = gate + r0 * g.ldx + 8 * c;
        const uint16_t* upp = up + r0 * g.ldx + 8 * c;
        for (int64_t r = r0; r < r1; ++r) {
            uint32_t h[4];
            swiglu8(ld16(gp), ld16(upp), h);
#pragma unroll
            for (int k = 0; k < 4; ++k) m2 = pk_max_u16(m2, mag2(h[k]));
            gp += g.ldx;
            upp += g.ldx;
        }
    }
    reduce_and_finish(fold_max(m2), ws, tensor_scale, amax_out);
}

__global__ __launch_bounds__(1024) void swiglu_pack_kernel(const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ up, RowGeo g,
                                                           const float* tensor_scale,
                                                           uint8_t* __restrict__ qdata,
                                                           uint8_t* __restrict__ sfa, int reverse) {
    const float s_g = tensor_scale[0];
    const bool sg_fast = scale_in_fast_range(s_g);
    const float rg = 1.0f / s_g;
    const int64_t tile = reverse ? (int64_t)(gridDim.x - 1 - blockIdx.x) : (int64_t)blockIdx.x;
    const int64_t r0 = tile * g.rows_per_wg;
    const int64_t r1 = r0 + g.rows_per_wg < g.rows_total ? r0 + g.rows_per_wg : g.rows_total;
    const int64_t qld = 4 * (int64_t)g.C8, sld = g.C8 >> 1;
    for (int j = 0; j < g.J; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c >= g.C8) break;
        const int64_t rm = r1 < g.M ? r1 : g.M;
        const uint16_t* gp = gate + r0 * g.ldx + 8 * c;
        const uint16_t* upp = up + r0 * g.ldx + 8 * c;
        for (int64_t r = r0; r < rm; ++r) {
            uint32_t h[4];
            swiglu8(ld16(gp), ld16(upp), h);
            pack_block_store(h, s_g, rg, sg_fast, qdata + r * qld, sfa + r * sld, c);
            gp += g.ldx;
            upp += g.ldx;
        }
        for (int64_t r = (r0 > g.M ? r0 : g.M); r < r1; ++r) {
            *reinterpret_cast<uint32_t*>(qdata + r * qld + 4 * c) = 0u;
            if ((c & 1) == 0) sfa[r * sld + (c >> 1)] = 0;
        }
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

__global__ void step_swiglu_kernel(const uint16_t* g, const uint16_t* u, uint16_t* h, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        h[i] = (uint16_t)(swiglu2((uint32_t)g[i], (uint32_t)u[i]) & 0xFFFF);
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
                                  float* tensor_scale, float* amax_out, hipStream_t s) {
    hipLaunchKernelGGL(modulate_absmax_kernel, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, ws, tensor_scale,
                       amax_out);
    return hipGetLastError();
}

hipError_t launch_modulate_pack(const uint16_t* x, const RowGeo& g, const SegParams& seg, const float* tensor_scale,
                                uint8_t* qdata, uint8_t* sfa, hipStream_t s) {
    hipLaunchKernelGGL(modulate_pack_kernel, dim3(g.grid), dim3(g.block), 0, s, x, g, seg, tensor_scale, qdata, sfa,
                       g.reverse);
    return hipGetLastError();
}

hipError_t launch_swiglu_absmax(const uint16_t* gate, const uint16_t* up, const RowGeo& g, uint32_t* ws,
                                float* tensor_scale, float* amax_out, hipStream_t s) {
    hipLaunchKernelGGL(swiglu_absmax_kernel, dim3(g.grid), dim3(g.block), 0, s, gate, up, g, ws, tensor_scale,
                       amax_out);
    return hipGetLastError();
}

hipError_t launch_swiglu_pack(const uint16_t* gate, const uint16_t* up, const RowGeo& g, const float* tensor_scale,
                              uint8_t* qdata, uint8_t* sfa, hipStream_t s) {
    hipLaunchKernelGGL(swiglu_pack_kernel, dim3(g.grid), dim3(g.block), 0, s, gate, up, g, tensor_scale, qdata, sfa,
                       g.reverse);
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
