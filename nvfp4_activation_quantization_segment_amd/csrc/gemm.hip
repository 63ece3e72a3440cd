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
// Tiling.  A workgroup of 8 waves (two per SIMD) computes a 256x256 output
// tile; each wave a 128(M) x 64(N) sub-tile as 4x2 v_mfma_f32_32x32x16_f16
// tiles with 128 fp32 accumulators per lane.  Every packed element is decoded
// once per workgroup: thread t < 256 decodes activation row t, thread t >= 256
// weight row t-256, 64 values per K step of 64, into double-buffered fp16
// tiles in LDS (256 rows x 64, row stride 144 bytes so that the 32 rows one
// MFMA fragment reads fall on distinct bank groups); the waves then read their
// fragments with 16-byte LDS loads.  The MFMA A operand is the weight (rows
// n) and the B operand the activation (rows m), so each lane's accumulators
// hold four consecutive n of one m and the epilogue stores 8 contiguous bytes.
// Two waves per SIMD let the hardware overlap one wave's decode and LDS work
// with the other's MFMAs.
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 64, kWM = 128, kWN = 64;

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

// LDS tiles: decoded fp16 [256 rows][64 k] per operand, row stride 72 halves
// (144 bytes: 16 bytes of padding make the 32 rows read by one MFMA fragment
// fall on distinct bank groups), two stages.
constexpr int kLDK = kBK + 8;
constexpr int kTileHalves = kBM * kLDK;  // per operand per stage
constexpr int kLdsBytes = 2 /*stages*/ * 2 /*operands*/ * kTileHalves * 2;

struct RowPack {
    uint4 q0, q1;  // 64 nibbles of one row for one K step
    uint32_t sc;   // its 4 block scales
};

__device__ __forceinline__ RowPack load_row(const uint8_t* q, const uint8_t* sf, uint32_t qoff, uint32_t soff) {
    RowPack r;
    r.q0 = *reinterpret_cast<const uint4*>(q + qoff);
    r.q1 = *reinterpret_cast<const uint4*>(q + qoff + 16);
    r.sc = *reinterpret_cast<const uint32_t*>(sf + soff);
    return r;
}

// Decode one row's 64 values into LDS (8 x 16-byte stores).
__device__ __forceinline__ void store_row(const RowPack& r, _Float16* dst) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t w = word_of(i < 4 ? r.q0 : r.q1, i & 3);
        const f16x8 v = decode8(w, sf_raw2(r.sc, i >> 1));
        *reinterpret_cast<f16x8*>(dst + 8 * i) = v;
    }
}

// Decode words 2p and 2p+1 of a staged row (the 16 values of block p) into
// LDS: two 16-byte stores.
__device__ __forceinline__ void store_part(const RowPack& r, int p, _Float16* dst) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 2 * p + u;
        const uint32_t w = word_of(i < 4 ? r.q0 : r.q1, i & 3);
        *reinterpret_cast<f16x8*>(dst + 8 * i) = decode8(w, sf_raw2(r.sc, i >> 1));
    }
}

// One K step on LDS buffer CUR, in four phases (one per 16-wide K slice j):
// read the fragments of slice j+1, decode a quarter of this thread's row of the
// next stage (DECODE) into the other buffer, and issue the 8 MFMAs of slice j.
// CUR is a template parameter so that both buffers' offsets are constants and
// the reads of one buffer and the writes of the other are visibly independent.
// The packed row of the stage after next is fetched at the start of the step.
template <int CUR, bool DECODE>
__device__ __forceinline__ void k_step(_Float16* __restrict__ lds, f32x16 (&acc)[2][4], RowPack& ra,
                                       const GemmArgs& a, uint32_t roff, uint32_t rso, const uint8_t* q,
                                       const uint8_t* sf, int next_stage, int tid, int wrow0, int arow0, int h) {
    const _Float16* cA = lds + CUR * kTileHalves;
    const _Float16* cW = lds + (2 + CUR) * kTileHalves;
    // thread tid < 256 decodes activation row tid, else weight row tid-256
    _Float16* dst = lds + ((tid < 256 ? 0 : 2) + (CUR ^ 1)) * kTileHalves + (tid & 255) * kLDK;
    RowPack na;
    if (DECODE) {
        const uint32_t db = 32u * next_stage, ds = 4u * next_stage;
        na = load_row(q, sf, roff + db, rso + ds);
    }
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
        if (DECODE) store_part(ra, j, dst);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc[i][k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[b][i], af[b][k], acc[i][k], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (DECODE) ra = na;
    __syncthreads();
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void
gemm_kernel(GemmArgs a, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) _Float16 lds[kLdsBytes / 2];

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

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int h = lane >> 5, l32 = lane & 31;
    const uint32_t Kb = (uint32_t)a.K >> 1, Ks = (uint32_t)a.K >> 4;
    const uint8_t* q = tid < 256 ? a.qa : a.qw;
    const uint8_t* sf = tid < 256 ? a.sfa : a.sfw;
    int row;
    if (tid < 256) { row = tm * kBM + tid; row = row < a.M_pad ? row : a.M_pad - 1; }
    else { row = tn * kBN + (tid - 256); row = row < a.N ? row : a.N - 1; }
    const uint32_t roff = (uint32_t)row * Kb, rso = (uint32_t)row * Ks;

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = (f32x16){0};
    const int wrow0 = wn * 64 + l32;
    const int arow0 = wm * 128 + l32;
    const int nit = a.K / kBK;
    RowPack ra = load_row(q, sf, roff, rso);
    store_row(ra, lds + (tid < 256 ? 0 : 2) * kTileHalves + (tid & 255) * kLDK);
    {
        const int s1 = nit > 1 ? 1 : 0;
        ra = load_row(q, sf, roff + 32u * s1, rso + 4u * s1);
    }
    __syncthreads();
    int it = 0;
    for (; it + 2 <= nit - 1; it += 2) {
        const int n2 = it + 2 < nit ? it + 2 : nit - 1;
        const int n3 = it + 3 < nit ? it + 3 : nit - 1;
        k_step<0, true>(lds, acc, ra, a, roff, rso, q, sf, n2, tid, wrow0, arow0, h);
        k_step<1, true>(lds, acc, ra, a, roff, rso, q, sf, n3, tid, wrow0, arow0, h);
    }
    if (it < nit - 1) {
        k_step<0, true>(lds, acc, ra, a, roff, rso, q, sf, nit - 1, tid, wrow0, arow0, h);
        ++it;
    }
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
                for (int k = 0; k < 4; ++k)
                    acc[i][k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[i], af[k], acc[i][k], 0, 0, 0);
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
        for (int i = 0; i < 2; ++i) {
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
    hipLaunchKernelGGL(gemm_kernel, dim3(tiles_m * tiles_n), dim3(512), 0, s, a, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace nvfp4
