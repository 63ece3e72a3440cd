// NVFP4 block-scaled GEMM for gfx950:  out = bf16(alpha * A W^T).
//
// Operation ("FC2 NVFP4 Library Scheduling", Exact Operation): row-major packed
// activation [M,K] times packed weight [N,K] -> BF16 [M,N], FP32 accumulation,
// alpha = activation tensor scale * weight tensor scale applied before the
// BF16 conversion ("NVFP4 Streaming Design", P0).
//
// Decode.  Every E2M1 value times an E4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16; products of two such fp16
// values are exact in fp32.  The MFMA path is therefore f16 (same dense rate
// as bf16 on gfx950) with exact operands; only the fp32 accumulation order
// differs from an exact dot product.  A nibble pair decodes with one
// v_cvt_scalef32_pk_f16_fp4 (scale 256, a power of two, which the
// instruction applies exactly) followed by one v_pk_mul_f16 by the raw E4M3
// bits reinterpreted as fp16 (equal to sf * 2^-8, subnormals included).
//
// Tiling.  A workgroup of 4 waves computes a 256x256 output tile; each wave a
// 128x128 sub-tile as 4x4 v_mfma_f32_32x32x16_f16 tiles with 256 fp32
// accumulators per lane.  The MFMA A operand is the weight (rows n) and the
// B operand the activation (rows m), so each lane's accumulators hold four
// consecutive n of one m and the epilogue stores 8 contiguous bytes.  Packed
// data goes straight from global memory to registers: per K step of 64 a lane
// reads 16 bytes (32 nibbles) of each of its 4 weight and 4 activation rows
// and one 4-byte word of their scales; the K order inside the step is
// permuted identically for both operands, which leaves the sum unchanged.
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 64, kWM = 128, kWN = 128;

// Raw E4M3 bits of byte `b` of a scale word, as two fp16 equal to sf * 2^-8.
__device__ __forceinline__ uint32_t sf_raw2(uint32_t word, int b) {
    return ((word >> (8 * b)) & 0x7Fu) * 0x00800080u;
}

// 8 nibbles (element 2i in the low nibble of byte i) times the block scale.
__device__ __forceinline__ f16x8 decode8(uint32_t w, uint32_t sraw2) {
    const f16x2 s = __builtin_bit_cast(f16x2, sraw2);
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
    return (f16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
gemm_kernel(GemmArgs a, int tiles_m, int tiles_n) {
    // Tile order: each XCD (workgroups are dealt round-robin over 8) takes a
    // contiguous range of tiles, walked in groups of 8 M-tiles so that the
    // workgroups resident on one XCD share activation and weight rows in L2.
    const int T = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int per = T / 8;
    const int logical = (bid < per * 8) ? (bid % 8) * per + bid / 8 : bid;
    constexpr int GM = 8;
    const int gsz = GM * tiles_n;
    const int first_m = (logical / gsz) * GM;
    const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int tm = first_m + (logical % gsz) % gm;
    const int tn = (logical % gsz) / gm;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const uint32_t Kb = (uint32_t)a.K >> 1, Ks = (uint32_t)a.K >> 4;

    uint32_t woff[4], aoff[4], wso[4], aso[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int n = tn * kBN + wn * kWN + i * 32 + l32;
        n = n < a.N ? n : a.N - 1;
        int m = tm * kBM + wm * kWM + i * 32 + l32;
        m = m < a.M_pad ? m : a.M_pad - 1;
        woff[i] = (uint32_t)n * Kb + 16u * h;
        aoff[i] = (uint32_t)m * Kb + 16u * h;
        wso[i] = (uint32_t)n * Ks;
        aso[i] = (uint32_t)m * Ks;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = (f32x16){0};

    const int nit = a.K / kBK;
    uint4 wq[4], aq[4];
    uint32_t wsc[4], asc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wq[i] = *reinterpret_cast<const uint4*>(a.qw + woff[i]);
        aq[i] = *reinterpret_cast<const uint4*>(a.qa + aoff[i]);
        wsc[i] = *reinterpret_cast<const uint32_t*>(a.sfw + wso[i]);
        asc[i] = *reinterpret_cast<const uint32_t*>(a.sfa + aso[i]);
    }

    for (int it = 0; it < nit; ++it) {
        uint4 wqn[4], aqn[4];
        uint32_t wscn[4], ascn[4];
        if (it + 1 < nit) {
            const uint32_t db = 32u * (it + 1), ds = 4u * (it + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wqn[i] = *reinterpret_cast<const uint4*>(a.qw + woff[i] + db);
                aqn[i] = *reinterpret_cast<const uint4*>(a.qa + aoff[i] + db);
                wscn[i] = *reinterpret_cast<const uint32_t*>(a.sfw + wso[i] + ds);
                ascn[i] = *reinterpret_cast<const uint32_t*>(a.sfa + aso[i] + ds);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 2 * h + (j >> 1);
            f16x8 wf[4], af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wf[i] = decode8(word_of(wq[i], j), sf_raw2(wsc[i], b));
                af[i] = decode8(word_of(aq[i], j), sf_raw2(asc[i], b));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    acc[i][k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[i], af[k], acc[i][k], 0, 0, 0);
        }
        if (it + 1 < nit) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wq[i] = wqn[i];
                aq[i] = aqn[i];
                wsc[i] = wscn[i];
                asc[i] = ascn[i];
            }
        }
    }

    // Epilogue: alpha = RN(s_a * s_w) applied in fp32, then bf16 (nearest-even).
    const float alpha = a.a_scale[0] * a.w_scale[0];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int m = tm * kBM + wm * kWM + k * 32 + l32;
        if (m >= a.M) continue;
        uint16_t* orow = a.out + (int64_t)m * a.ldo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = tn * kBN + wn * kWN + i * 32 + 8 * q + 4 * h;
                if (n >= a.N) continue;
                const f32x16& c = acc[i][k];
                uint2 v;
                v.x = pack_bf16x2(c[4 * q + 0] * alpha, c[4 * q + 1] * alpha);
                v.y = pack_bf16x2(c[4 * q + 2] * alpha, c[4 * q + 3] * alpha);
                *reinterpret_cast<uint2*>(orow + n) = v;
            }
        }
    }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
    const int tiles_m = (a.M + kBM - 1) / kBM;
    const int tiles_n = (a.N + kBN - 1) / kBN;
    hipLaunchKernelGGL(gemm_kernel, dim3(tiles_m * tiles_n), dim3(256), 0, s, a, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace nvfp4
