// Internal declarations shared by the API layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

// Segment table passed to the kernels by value.
struct SegParams {
    int32_t count;
    int64_t row_start[NVFP4_MAX_SEGMENTS + 1];
    const uint16_t* shift;
    const uint16_t* scale;
    int64_t ld;
};

// Row-pass geometry: each thread owns column chunks c = threadIdx.x + j*block
// (j < J) of 8 columns in the absmax passes and 16 (one block) in the pack
// passes; workgroup b visits rows b, b+grid, b+2*grid, ... (grid-stride), or
// in the pack passes R rows per iteration when a row is short.
struct RowGeo {
    int64_t M;            // logical rows
    int64_t rows_total;   // rows the grid covers (M, or M_pad when padding is written)
    int64_t ldx;          // input row stride (elements)
    int32_t C8;           // 8-column chunks per row
    int32_t J;            // chunks per thread (of the pass's chunk width)
    int32_t grid;
    int32_t block;
    int32_t reverse;      // the pass visits rows last-to-first
    int32_t R;            // rows per workgroup iteration (pack passes; 1 for absmax)
};

enum StepKind { STEP_MODULATE, STEP_SWIGLU, STEP_BLOCK_SCALE, STEP_ELEMENT_CODE, STEP_E2M1, STEP_E4M3 };

hipError_t launch_modulate_absmax(const uint16_t* x, const RowGeo& g, const SegParams& seg, uint32_t* ws,
                                  float* tensor_scale, float* amax_out, bool plain, hipStream_t s);
hipError_t launch_modulate_pack(const uint16_t* x, const RowGeo& g, const SegParams& seg, const float* tensor_scale,
                                uint8_t* qdata, uint8_t* sfa, bool plain, hipStream_t s);
// Single-pass producer: one launch of at most modulate_quantize_grid()
// workgroups, as many as the device holds at once (0 when that cannot be
// determined).  The workspace holds 256 header bytes, then one 8-byte arrival
// word and one 8-byte claim word per workgroup.
constexpr int kMaxDevices = 32;
constexpr int kMaxGridSlots = 1024;
constexpr size_t kWorkspaceBytes = 256 + 2 * 8 * kMaxGridSlots;
// Per launch: a tag no earlier launch used (44 bits, not 0), the bound on the
// grid-barrier wait and the wait after which a workgroup starts computing the
// pass 1 of workgroups that have not arrived, both in ticks of the 100 MHz
// real-time counter.
struct BarrierArgs {
    uint64_t tag;
    uint64_t wait_ticks;
    uint64_t help_ticks;
};
BarrierArgs next_barrier_args();
int modulate_quantize_grid();
// plain: the plain quantizer (y = x; seg is not read).
hipError_t launch_modulate_quantize(const uint16_t* x, const RowGeo& g, const SegParams& seg, uint32_t* ws,
                                    float* tensor_scale, float* amax_out, uint8_t* qdata, uint8_t* sfa, bool plain,
                                    const BarrierArgs& ba, hipStream_t s);
// Both SwiGLU passes in one launch (after the silu table fill).
int swiglu_quantize_grid();
hipError_t launch_swiglu_quantize(const uint16_t* gate, const uint16_t* up, const RowGeo& g, uint32_t* ws,
                                  float* tensor_scale, float* amax_out, uint8_t* qdata, uint8_t* sfa,
                                  const BarrierArgs& ba, hipStream_t s);
// fill: enqueue the silu table fill first (each public entry point does once)
hipError_t launch_swiglu_absmax(const uint16_t* gate, const uint16_t* up, const RowGeo& g, uint32_t* ws,
                                float* tensor_scale, float* amax_out, bool fill, hipStream_t s);
hipError_t launch_swiglu_pack(const uint16_t* gate, const uint16_t* up, const RowGeo& g, const float* tensor_scale,
                              uint8_t* qdata, uint8_t* sfa, bool fill, hipStream_t s);
hipError_t launch_step(int which, const void* a, const void* b, const void* c, void* out, int64_t n, hipStream_t s);
// Zero-fills `bytes` (a multiple of 16, at most 16 x 65,536) of device memory
// with one small kernel on s.
hipError_t launch_clear_workspace(void* ws, size_t bytes, hipStream_t s);

struct GemmArgs {
    const uint8_t* qa;
    const uint8_t* sfa;
    const float* a_scale;
    const uint8_t* qw;
    const uint8_t* sfw;
    const float* w_scale;
    uint16_t* out;
    int64_t ldo;
    int32_t M, M_pad, N, K;
    // Residual epilogue (epi != 0): out = bf16(residual + bf16(gate[s][n] * o)),
    // s the segment of row m (row_start has nseg + 1 entries).
    int32_t epi;
    int32_t nseg;
    int32_t row_start[NVFP4_MAX_SEGMENTS + 1];
    const uint16_t* gate;
    int64_t ld_gate;
    const uint16_t* residual;
    int64_t ldr;
};
// Tiles of one GEMM launch (see gemm.hip).
struct GemmPart {
    int32_t tiles_m, tiles_n;
    int32_t tile_base;  // first logical tile of a split launch
    int32_t tiles;      // tiles of the launch (main) or tail tiles (split)
    int32_t ksplit;     // K pieces per tail tile
    int32_t ks;         // K steps (of 64) per piece
    float* partial;     // fp32 partial sums of the tail pieces
};
// How a GEMM is cut: `full` tiles over all of K, then `tail` tiles in
// `ksplit` K pieces of `ks` steps, summed by a finalize kernel.
struct GemmPlan {
    int tiles_m, tiles_n, full, tail, ksplit, ks;
    size_t workspace_bytes;
};
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const GemmArgs& a, float* workspace, bool split, hipStream_t s);

}  // namespace nvfp4
