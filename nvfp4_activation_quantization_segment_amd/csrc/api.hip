// C ABI of the NVFP4 producer and GEMM: argument validation, launch geometry
// and error reporting.  Every check happens before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "internal.h"

using namespace nvfp4;

namespace {

thread_local int g_last_hip_error = 0;

nvfp4_status hip_status(hipError_t e) {
    if (e == hipSuccess) return NVFP4_OK;
    g_last_hip_error = (int)e;
    return NVFP4_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Tags of the single launches: one process-wide counter, so that no two
// launches on any workspace share one (words of earlier launches then never
// match), and the wait bound in microseconds.
std::atomic<uint64_t> g_barrier_tag{0};
std::atomic<uint64_t> g_barrier_wait_us{1000000};
std::atomic<uint64_t> g_barrier_help_us{100};

int64_t pad64(int64_t m) { return (m + 63) / 64 * 64; }

// Geometry of a row pass over [rows_total, width] with 8-column chunks.
// cols_per_thread: 8 (absmax passes) or 16 (pack passes, one block per thread).
RowGeo row_geo(int64_t M, int64_t rows_total, int64_t width, int64_t ld, int target_wgs, int reverse,
               int cols_per_thread) {
    RowGeo g;
    g.M = M;
    g.rows_total = rows_total;
    g.ldx = ld;
    g.C8 = (int32_t)(width / 8);
    const int chunks = (int)(width / cols_per_thread);
    g.J = (chunks + 1023) / 1024;
    const int per = (chunks + g.J - 1) / g.J;
    // pack passes put several short rows in one workgroup so that few lanes idle
    g.R = (cols_per_thread == 16 && chunks <= 512) ? 1024 / chunks : 1;
    g.block = (per * g.R + 63) / 64 * 64;
    // rows are visited grid-stride; the grid never exceeds the row-group count
    const int64_t groups = (rows_total + g.R - 1) / g.R;
    const int64_t grid = groups < target_wgs ? groups : target_wgs;
    g.grid = (int32_t)(grid > 0 ? grid : 1);
    g.reverse = reverse;
    return g;
}

// Grid sizes (rows are visited grid-stride).  The absmax passes end with one
// atomic per workgroup, so fewer, wider workgroups are best there.
constexpr int kAbsmaxWgs = 256;
constexpr int kPackWgs = 1024;
// The SwiGLU passes hold a 128 KB table in LDS: one workgroup per CU.
constexpr int kSwigluPackWgs = 256;
// The ring's chunk packs run in the gaps the GEMMs leave: few, long workgroups.
constexpr int kRingPackWgs = 256;

nvfp4_status check_segments(const nvfp4_segments* seg, int64_t M, int64_t D, SegParams* out) {
    if (!seg || !seg->row_start || !seg->shift || !seg->scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (seg->count < 1 || seg->count > NVFP4_MAX_SEGMENTS) return NVFP4_ERR_SEGMENTS;
    if (seg->row_start[0] != 0 || seg->row_start[seg->count] != M) return NVFP4_ERR_SEGMENTS;
    for (int s = 0; s < seg->count; ++s)
        if (seg->row_start[s + 1] <= seg->row_start[s]) return NVFP4_ERR_SEGMENTS;
    if (seg->ld < D) return NVFP4_ERR_INVALID_ARGUMENT;
    if (seg->ld % 8 != 0 || !aligned(seg->shift, 16) || !aligned(seg->scale, 16)) return NVFP4_ERR_ALIGNMENT;
    memset(out, 0, sizeof(*out));
    out->count = seg->count;
    for (int s = 0; s <= seg->count; ++s) out->row_start[s] = seg->row_start[s];
    out->shift = seg->shift;
    out->scale = seg->scale;
    out->ld = seg->ld;
    return NVFP4_OK;
}

nvfp4_status check_rows(const void* x, int64_t M, int64_t D, int64_t ld) {
    if (!x) return NVFP4_ERR_INVALID_ARGUMENT;
    if (M <= 0 || D <= 0) return NVFP4_ERR_INVALID_ARGUMENT;
    if (D % 16 != 0) return NVFP4_ERR_SHAPE;
    if (D / 8 > (int64_t)1 << 20) return NVFP4_ERR_SHAPE;
    if (ld < D) return NVFP4_ERR_INVALID_ARGUMENT;
    if (ld % 8 != 0 || !aligned(x, 16)) return NVFP4_ERR_ALIGNMENT;
    return NVFP4_OK;
}

nvfp4_status check_outputs(const uint8_t* qdata, const uint8_t* sfa, int64_t M, int64_t M_pad) {
    if (!qdata || !sfa) return NVFP4_ERR_INVALID_ARGUMENT;
    if (M_pad < pad64(M)) return NVFP4_ERR_SHAPE;
    if (!aligned(qdata, 4)) return NVFP4_ERR_ALIGNMENT;
    return NVFP4_OK;
}

// The barrier words of nvfp4_modulate_quantize_noalloc: a fixed array in the
// code object, one copy on every device the library runs on, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): it passes the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kWorkspaceBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device.
nvfp4_status scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return NVFP4_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NVFP4_OK;
}

}  // namespace

BarrierArgs nvfp4::next_barrier_args() {
    constexpr uint64_t kTagMask = ((uint64_t)1 << 44) - 1;
    uint64_t t = (g_barrier_tag.fetch_add(1) + 1) & kTagMask;
    if (t == 0) t = (g_barrier_tag.fetch_add(1) + 1) & kTagMask;
    BarrierArgs ba;
    ba.tag = t;
    const auto ticks = [](uint64_t us) { return us > UINT64_MAX / 100 ? UINT64_MAX : us * 100; };  // 100 MHz
    ba.wait_ticks = ticks(g_barrier_wait_us.load());
    ba.help_ticks = ticks(g_barrier_help_us.load());
    return ba;
}

extern "C" {

uint64_t nvfp4_set_barrier_timeout_us(uint64_t microseconds) { return g_barrier_wait_us.exchange(microseconds); }

uint64_t nvfp4_set_barrier_help_us(uint64_t microseconds) { return g_barrier_help_us.exchange(microseconds); }

int64_t nvfp4_padded_rows(int64_t m) { return m <= 0 ? 0 : pad64(m); }

size_t nvfp4_absmax_workspace_bytes(void) { return kWorkspaceBytes; }

const char* nvfp4_status_string(nvfp4_status s) {
    switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARGUMENT: return "invalid argument";
    case NVFP4_ERR_SHAPE: return "unsupported shape";
    case NVFP4_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case NVFP4_ERR_SEGMENTS: return "invalid segment table";
    case NVFP4_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

int nvfp4_last_hip_error(void) { return g_last_hip_error; }

nvfp4_status nvfp4_modulate_absmax(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                   const nvfp4_segments* seg, void* workspace, float* tensor_scale,
                                   float* amax_out, void* stream) {
    nvfp4_status st = check_rows(x, M, D, ldx);
    if (st != NVFP4_OK) return st;
    SegParams sp;
    if ((st = check_segments(seg, M, D, &sp)) != NVFP4_OK) return st;
    if (!workspace || !tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 4) || !aligned(tensor_scale, 4) || !aligned(amax_out, 4)) return NVFP4_ERR_ALIGNMENT;
    const RowGeo g = row_geo(M, M, D, ldx, kAbsmaxWgs, 0, 8);
    return hip_status(launch_modulate_absmax(x, g, sp, (uint32_t*)workspace, tensor_scale, amax_out, false,
                                             (hipStream_t)stream));
}

nvfp4_status nvfp4_modulate_pack(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                 const nvfp4_segments* seg, const float* tensor_scale, uint8_t* qdata,
                                 uint8_t* sfa, int64_t M_pad, void* stream) {
    nvfp4_status st = check_rows(x, M, D, ldx);
    if (st != NVFP4_OK) return st;
    SegParams sp;
    if ((st = check_segments(seg, M, D, &sp)) != NVFP4_OK) return st;
    if (!tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(tensor_scale, 4)) return NVFP4_ERR_ALIGNMENT;
    if ((st = check_outputs(qdata, sfa, M, M_pad)) != NVFP4_OK) return st;
    const RowGeo g = row_geo(M, M_pad, D, ldx, kPackWgs, 1, 16);
    return hip_status(launch_modulate_pack(x, g, sp, tensor_scale, qdata, sfa, false, (hipStream_t)stream));
}

// Both passes, as one launch where it applies, else as the two passes; the
// plain quantizer passes plain = true and a segment table that is never read.
static nvfp4_status quantize_both(const uint16_t* x, int64_t M, int64_t D, int64_t ldx, const SegParams& sp,
                                  bool plain, void* workspace, float* tensor_scale, float* amax_out,
                                  uint8_t* qdata, uint8_t* sfa, int64_t M_pad, hipStream_t s) {
    // one launch when a row fits one workgroup (D <= 16384) and every byte
    // offset into x, qdata and sfa fits 32 bits
    const bool off32 = ((M - 1) * ldx + D) * 2 < ((int64_t)1 << 32) && M_pad * (D / 2) < ((int64_t)1 << 32);
    const int G = (D / 16 <= 1024 && off32) ? modulate_quantize_grid() : 0;
    if (G > 0) {
        const RowGeo g = row_geo(M, M_pad, D, ldx, G, 1, 16);
        return hip_status(launch_modulate_quantize(x, g, sp, (uint32_t*)workspace, tensor_scale, amax_out, qdata,
                                                   sfa, plain, next_barrier_args(), s));
    }
    nvfp4_status st;
    const RowGeo g1 = row_geo(M, M, D, ldx, kAbsmaxWgs, 0, 8);
    if ((st = hip_status(launch_modulate_absmax(x, g1, sp, (uint32_t*)workspace, tensor_scale, amax_out, plain, s))) !=
        NVFP4_OK)
        return st;
    const RowGeo g2 = row_geo(M, M_pad, D, ldx, kPackWgs, 1, 16);
    return hip_status(launch_modulate_pack(x, g2, sp, tensor_scale, qdata, sfa, plain, s));
}

nvfp4_status nvfp4_modulate_quantize(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                     const nvfp4_segments* seg, void* workspace, float* tensor_scale,
                                     float* amax_out, uint8_t* qdata, uint8_t* sfa, int64_t M_pad, void* stream) {
    nvfp4_status st = check_rows(x, M, D, ldx);
    if (st != NVFP4_OK) return st;
    SegParams sp;
    if ((st = check_segments(seg, M, D, &sp)) != NVFP4_OK) return st;
    if (!workspace || !tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 4) || !aligned(tensor_scale, 4) || !aligned(amax_out, 4)) return NVFP4_ERR_ALIGNMENT;
    if ((st = check_outputs(qdata, sfa, M, M_pad)) != NVFP4_OK) return st;
    return quantize_both(x, M, D, ldx, sp, false, workspace, tensor_scale, amax_out, qdata, sfa, M_pad,
                         (hipStream_t)stream);
}

nvfp4_status nvfp4_modulate_quantize_noalloc(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                             const nvfp4_segments* seg, float* tensor_scale, float* amax_out,
                                             uint8_t* qdata, uint8_t* sfa, int64_t M_pad, void* stream) {
    nvfp4_status st = check_rows(x, M, D, ldx);
    if (st != NVFP4_OK) return st;
    SegParams sp;
    if ((st = check_segments(seg, M, D, &sp)) != NVFP4_OK) return st;
    if (!tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(tensor_scale, 4) || !aligned(amax_out, 4)) return NVFP4_ERR_ALIGNMENT;
    if ((st = check_outputs(qdata, sfa, M, M_pad)) != NVFP4_OK) return st;
    // the barrier needs 256 header bytes and 16 bytes per workgroup; the grid
    // is capped at kMaxGridSlots, so every accepted shape fits the scratch
    const size_t need = 256 + 16 * (size_t)kMaxGridSlots;
    if (need > sizeof(scratch)) return NVFP4_ERR_SHAPE;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != NVFP4_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    if ((st = hip_status(launch_clear_workspace(ws, need, s))) != NVFP4_OK) return st;
    return quantize_both(x, M, D, ldx, sp, false, ws, tensor_scale, amax_out, qdata, sfa, M_pad, s);
}

nvfp4_status nvfp4_quantize(const uint16_t* x, int64_t M, int64_t D, int64_t ldx, void* workspace,
                            float* tensor_scale, float* amax_out, uint8_t* qdata, uint8_t* sfa, int64_t M_pad,
                            void* stream) {
    nvfp4_status st = check_rows(x, M, D, ldx);
    if (st != NVFP4_OK) return st;
    if (!workspace || !tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 4) || !aligned(tensor_scale, 4) || !aligned(amax_out, 4)) return NVFP4_ERR_ALIGNMENT;
    if ((st = check_outputs(qdata, sfa, M, M_pad)) != NVFP4_OK) return st;
    SegParams sp;  // one segment over all rows; its parameters are never read
    memset(&sp, 0, sizeof(sp));
    sp.count = 1;
    sp.row_start[1] = M;
    return quantize_both(x, M, D, ldx, sp, true, workspace, tensor_scale, amax_out, qdata, sfa, M_pad,
                         (hipStream_t)stream);
}

nvfp4_status nvfp4_swiglu_absmax(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F, int64_t ld,
                                 void* workspace, float* tensor_scale, float* amax_out, void* stream) {
    nvfp4_status st = check_rows(gate, M, F, ld);
    if (st != NVFP4_OK) return st;
    if ((st = check_rows(up, M, F, ld)) != NVFP4_OK) return st;
    if (!workspace || !tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 4) || !aligned(tensor_scale, 4) || !aligned(amax_out, 4)) return NVFP4_ERR_ALIGNMENT;
    const RowGeo g = row_geo(M, M, F, ld, kAbsmaxWgs, 0, 8);
    return hip_status(launch_swiglu_absmax(gate, up, g, (uint32_t*)workspace, tensor_scale, amax_out, true,
                                           (hipStream_t)stream));
}

nvfp4_status nvfp4_swiglu_pack(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F, int64_t ld,
                               const float* tensor_scale, uint8_t* qdata, uint8_t* sfa, int64_t M_pad,
                               void* stream) {
    nvfp4_status st = check_rows(gate, M, F, ld);
    if (st != NVFP4_OK) return st;
    if ((st = check_rows(up, M, F, ld)) != NVFP4_OK) return st;
    if (!tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(tensor_scale, 4)) return NVFP4_ERR_ALIGNMENT;
    if ((st = check_outputs(qdata, sfa, M, M_pad)) != NVFP4_OK) return st;
    const RowGeo g = row_geo(M, M_pad, F, ld, kSwigluPackWgs, 1, 16);
    return hip_status(launch_swiglu_pack(gate, up, g, tensor_scale, qdata, sfa, true, (hipStream_t)stream));
}

nvfp4_status nvfp4_swiglu_quantize(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F, int64_t ld,
                                   void* workspace, float* tensor_scale, float* amax_out, uint8_t* qdata,
                                   uint8_t* sfa, int64_t M_pad, void* stream) {
    nvfp4_status st = check_rows(gate, M, F, ld);
    if (st != NVFP4_OK) return st;
    if ((st = check_rows(up, M, F, ld)) != NVFP4_OK) return st;
    if (!workspace || !tensor_scale) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 4) || !aligned(tensor_scale, 4) || !aligned(amax_out, 4)) return NVFP4_ERR_ALIGNMENT;
    if ((st = check_outputs(qdata, sfa, M, M_pad)) != NVFP4_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    // one launch when a row fits one workgroup and every byte offset into
    // gate, up, qdata and sfa fits 32 bits
    const bool off32 = ((M - 1) * ld + F) * 2 < ((int64_t)1 << 32) && M_pad * (F / 2) < ((int64_t)1 << 32);
    const int G = (F / 16 <= 1024 && off32) ? swiglu_quantize_grid() : 0;
    if (G > 0) {
        const RowGeo g = row_geo(M, M_pad, F, ld, G, 1, 16);
        return hip_status(
            launch_swiglu_quantize(gate, up, g, (uint32_t*)workspace, tensor_scale, amax_out, qdata, sfa,
                                   next_barrier_args(), s));
    }
    const RowGeo g1 = row_geo(M, M, F, ld, kAbsmaxWgs, 0, 8);
    if ((st = hip_status(launch_swiglu_absmax(gate, up, g1, (uint32_t*)workspace, tensor_scale, amax_out, true, s))) !=
        NVFP4_OK)
        return st;
    const RowGeo g2 = row_geo(M, M_pad, F, ld, kSwigluPackWgs, 1, 16);
    return hip_status(launch_swiglu_pack(gate, up, g2, tensor_scale, qdata, sfa, false, s));
}

// Activation rows per launch: the chunk's packed rows stay below 2^32 bytes
// (the kernel's offsets are 32-bit and its loads are range-checked against
// 2^32 - 1), in whole 256-row tiles; 0 when K is too wide for even one tile
// (K > 2^25).
static int64_t gemm_chunk_rows(int64_t K) { return ((((int64_t)1 << 32) - 1) / (K / 2)) / 256 * 256; }

static nvfp4_status gemm_args(const uint8_t* qa, const uint8_t* sfa, const float* a_scale, int64_t M,
                              int64_t M_pad, const uint8_t* qw, const uint8_t* sfw, const float* w_scale, int64_t N,
                              int64_t K, uint16_t* out, int64_t ldo, GemmArgs* a) {
    if (!qa || !sfa || !a_scale || !qw || !sfw || !w_scale || !out) return NVFP4_ERR_INVALID_ARGUMENT;
    if (M <= 0 || N <= 0 || K <= 0 || ldo < N || M_pad < M) return NVFP4_ERR_INVALID_ARGUMENT;
    if (K % 64 != 0 || N % 16 != 0) return NVFP4_ERR_SHAPE;
    // 32-bit byte offsets inside the kernel: the weight must fit them; the
    // activation is launched in row chunks that do (run_gemm)
    if (N * (K / 2) >= ((int64_t)1 << 32) || gemm_chunk_rows(K) == 0) return NVFP4_ERR_SHAPE;
    if (M_pad >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
    if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(sfa, 4) || !aligned(sfw, 4) || !aligned(out, 8) ||
        ldo % 4 != 0 || !aligned(a_scale, 4) || !aligned(w_scale, 4))
        return NVFP4_ERR_ALIGNMENT;
    a->qa = qa;
    a->sfa = sfa;
    a->a_scale = a_scale;
    a->qw = qw;
    a->sfw = sfw;
    a->w_scale = w_scale;
    a->out = out;
    a->ldo = ldo;
    a->M = (int32_t)M;
    a->M_pad = (int32_t)M_pad;
    a->N = (int32_t)N;
    a->K = (int32_t)K;
    a->epi = 0;
    a->nseg = 0;
    memset(a->row_start, 0, sizeof(a->row_start));
    a->gate = nullptr;
    a->ld_gate = 0;
    a->residual = nullptr;
    a->ldr = 0;
    return NVFP4_OK;
}

// Workspace of the largest row chunk's plan (the chunks run in stream order
// and share it).
static size_t gemm_workspace(int64_t M, int64_t N, int64_t K) {
    const int64_t mc = gemm_chunk_rows(K);
    if (M <= mc) return gemm_plan(M, N, K).workspace_bytes;
    const size_t full = gemm_plan(mc, N, K).workspace_bytes;
    const int64_t last = M - (M - 1) / mc * mc;
    const size_t tail = gemm_plan(last, N, K).workspace_bytes;
    return full > tail ? full : tail;
}

// The GEMM as row chunks of gemm_chunk_rows(K): each launch sees its chunk's
// rows of qa, sfa, out and the residual from row 0, and the gate segment
// bounds shifted by the chunk's first row.
static nvfp4_status run_gemm(const GemmArgs& a, int64_t M, int64_t M_pad, void* workspace, bool use_ws,
                             hipStream_t s) {
    const int64_t mc = gemm_chunk_rows(a.K);
    for (int64_t r0 = 0; r0 < M; r0 += mc) {
        GemmArgs c = a;
        c.M = (int32_t)(M - r0 < mc ? M - r0 : mc);
        c.M_pad = (int32_t)(M_pad - r0 < mc ? M_pad - r0 : mc);
        c.qa = a.qa + r0 * (a.K / 2);
        c.sfa = a.sfa + r0 * (a.K / 16);
        c.out = a.out + r0 * a.ldo;
        if (a.epi) {
            c.residual = a.residual + r0 * a.ldr;
            for (int i = 0; i <= a.nseg; ++i) c.row_start[i] = (int32_t)(a.row_start[i] - r0);
        }
        const bool split = use_ws && gemm_plan(c.M, c.N, c.K).workspace_bytes > 0;
        const nvfp4_status st = hip_status(launch_gemm(c, split ? (float*)workspace : nullptr, split, s));
        if (st != NVFP4_OK) return st;
    }
    return NVFP4_OK;
}

nvfp4_status nvfp4_gemm(const uint8_t* qa, const uint8_t* sfa, const float* a_scale, int64_t M, int64_t M_pad,
                        const uint8_t* qw, const uint8_t* sfw, const float* w_scale, int64_t N, int64_t K,
                        uint16_t* out, int64_t ldo, void* stream) {
    GemmArgs a;
    const nvfp4_status st = gemm_args(qa, sfa, a_scale, M, M_pad, qw, sfw, w_scale, N, K, out, ldo, &a);
    if (st != NVFP4_OK) return st;
    return run_gemm(a, M, M_pad, nullptr, false, (hipStream_t)stream);
}

size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 64 != 0 || M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) ||
        K >= ((int64_t)1 << 31) || gemm_chunk_rows(K) == 0)
        return 0;
    return gemm_workspace(M, N, K);
}

nvfp4_status nvfp4_gemm_ws(const uint8_t* qa, const uint8_t* sfa, const float* a_scale, int64_t M, int64_t M_pad,
                           const uint8_t* qw, const uint8_t* sfw, const float* w_scale, int64_t N, int64_t K,
                           uint16_t* out, int64_t ldo, void* workspace, size_t workspace_bytes, void* stream) {
    GemmArgs a;
    const nvfp4_status st = gemm_args(qa, sfa, a_scale, M, M_pad, qw, sfw, w_scale, N, K, out, ldo, &a);
    if (st != NVFP4_OK) return st;
    const size_t need = gemm_workspace(M, N, K);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return NVFP4_ERR_INVALID_ARGUMENT;
        if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGNMENT;
    }
    return run_gemm(a, M, M_pad, workspace, need > 0, (hipStream_t)stream);
}

nvfp4_status nvfp4_gemm_gate_residual(const uint8_t* qa, const uint8_t* sfa, const float* a_scale, int64_t M,
                                      int64_t M_pad, const uint8_t* qw, const uint8_t* sfw, const float* w_scale,
                                      int64_t N, int64_t K, const nvfp4_row_gates* gates, const uint16_t* residual,
                                      int64_t ldr, uint16_t* out, int64_t ldo, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    GemmArgs a;
    nvfp4_status st = gemm_args(qa, sfa, a_scale, M, M_pad, qw, sfw, w_scale, N, K, out, ldo, &a);
    if (st != NVFP4_OK) return st;
    if (!gates || !gates->row_start || !gates->gate || !residual) return NVFP4_ERR_INVALID_ARGUMENT;
    if (gates->count < 1 || gates->count > NVFP4_MAX_SEGMENTS) return NVFP4_ERR_SEGMENTS;
    if (gates->row_start[0] != 0 || gates->row_start[gates->count] != M) return NVFP4_ERR_SEGMENTS;
    for (int s = 0; s < gates->count; ++s)
        if (gates->row_start[s + 1] <= gates->row_start[s]) return NVFP4_ERR_SEGMENTS;
    if (gates->ld < N || ldr < N) return NVFP4_ERR_INVALID_ARGUMENT;
    if (gates->ld % 4 != 0 || ldr % 4 != 0 || !aligned(gates->gate, 8) || !aligned(residual, 8))
        return NVFP4_ERR_ALIGNMENT;
    const size_t need = gemm_workspace(M, N, K);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return NVFP4_ERR_INVALID_ARGUMENT;
        if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGNMENT;
    }
    a.epi = 1;
    a.nseg = gates->count;
    for (int s = 0; s <= gates->count; ++s) a.row_start[s] = (int32_t)gates->row_start[s];
    a.gate = gates->gate;
    a.ld_gate = gates->ld;
    a.residual = residual;
    a.ldr = ldr;
    return run_gemm(a, M, M_pad, workspace, need > 0, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// Packed-tile ring ("NVFP4 Streaming Design", P2: N-group reuse through a
// bounded ring of packed activation slots, one full-activation scale reused
// by every chunk).  Host orchestration over three streams: the caller's
// stream runs pass 1 and the even chunks' GEMMs, one internal stream the
// chunk packs, another the odd chunks' GEMMs.  Events order every slot's
// reuse (a pack waits for the GEMM that last read its slot) and every GEMM
// (it waits for its chunk's pack), so no workgroup ever waits on another.
// Two GEMM streams let one chunk's GEMM fill the CUs that the previous
// chunk's last wave of tiles leaves idle, and the packs run in those gaps.
// ---------------------------------------------------------------------------
constexpr int kMaxRingSlots = 64;

struct RingState {
    bool ready = false;
    hipStream_t pack = nullptr, gemm_odd = nullptr;
    hipEvent_t start = nullptr, odd_done = nullptr;
    hipEvent_t packed[kMaxRingSlots] = {};
    hipEvent_t consumed[kMaxRingSlots] = {};
};
static RingState g_ring[kMaxDevices];
static std::mutex g_ring_mu[kMaxDevices];

static nvfp4_status ring_state(int dev, RingState** out) {
    RingState& r = g_ring[dev];
    if (!r.ready) {
        hipError_t e;
        if ((e = hipStreamCreateWithFlags(&r.pack, hipStreamNonBlocking)) != hipSuccess) return hip_status(e);
        if ((e = hipStreamCreateWithFlags(&r.gemm_odd, hipStreamNonBlocking)) != hipSuccess) return hip_status(e);
        if ((e = hipEventCreateWithFlags(&r.start, hipEventDisableTiming)) != hipSuccess) return hip_status(e);
        if ((e = hipEventCreateWithFlags(&r.odd_done, hipEventDisableTiming)) != hipSuccess) return hip_status(e);
        for (int i = 0; i < kMaxRingSlots; ++i) {
            if ((e = hipEventCreateWithFlags(&r.packed[i], hipEventDisableTiming)) != hipSuccess) return hip_status(e);
            if ((e = hipEventCreateWithFlags(&r.consumed[i], hipEventDisableTiming)) != hipSuccess)
                return hip_status(e);
        }
        r.ready = true;
    }
    *out = &r;
    return NVFP4_OK;
}

// Rows of every chunk's slot: chunk_rows (a multiple of 64), so that the last,
// shorter chunk's padding rows fit too.
static size_t ring_slot_bytes(int64_t chunk_rows, int64_t K) {
    return (size_t)chunk_rows * (size_t)(K / 2 + K / 16);
}

// K-split workspace of one chunk GEMM (the largest of a full and the last
// chunk), for each of the two GEMM streams.
static size_t ring_gemm_ws_half(int64_t M, int64_t chunk_rows, int64_t N, int64_t K) {
    const int64_t full = M < chunk_rows ? M : chunk_rows;
    const int64_t last = M - (M - 1) / chunk_rows * chunk_rows;
    const size_t a = gemm_workspace(full, N, K), b = gemm_workspace(last, N, K);
    const size_t w = a > b ? a : b;
    return (w + 255) / 256 * 256;
}

// The segment table restricted to rows [r0, r1), rebased to row 0.
static void chunk_segments(const SegParams& sp, int64_t r0, int64_t r1, SegParams* out) {
    memset(out, 0, sizeof(*out));
    int s0 = 0;
    while (sp.row_start[s0 + 1] <= r0) ++s0;
    int n = 0;
    out->row_start[0] = 0;
    for (int s = s0; s < sp.count && sp.row_start[s] < r1; ++s) {
        const int64_t hi = sp.row_start[s + 1] < r1 ? sp.row_start[s + 1] : r1;
        out->row_start[++n] = hi - r0;
    }
    out->count = n;
    out->shift = sp.shift + (int64_t)s0 * sp.ld;
    out->scale = sp.scale + (int64_t)s0 * sp.ld;
    out->ld = sp.ld;
}

static nvfp4_status ring_run(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const SegParams& sp,
                             void* workspace, float* tensor_scale, float* amax_out, uint8_t* ring, int slots,
                             int64_t chunk_rows, const GemmArgs& ga, uint8_t* gemm_ws, size_t ws_half,
                             hipStream_t s, RingState& rs) {
    nvfp4_status st;
    // pass 1 over every row: one tensor scale for all chunks
    const RowGeo g1 = row_geo(M, M, K, ldx, kAbsmaxWgs, 0, 8);
    if ((st = hip_status(launch_modulate_absmax(x, g1, sp, (uint32_t*)workspace, tensor_scale, amax_out, false,
                                                s))) != NVFP4_OK)
        return st;
    if ((st = hip_status(hipEventRecord(rs.start, s))) != NVFP4_OK) return st;
    if ((st = hip_status(hipStreamWaitEvent(rs.pack, rs.start, 0))) != NVFP4_OK) return st;
    if ((st = hip_status(hipStreamWaitEvent(rs.gemm_odd, rs.start, 0))) != NVFP4_OK) return st;
    const size_t slot_bytes = ring_slot_bytes(chunk_rows, K);
    const int64_t chunks = (M + chunk_rows - 1) / chunk_rows;
    for (int64_t c = 0; c < chunks; ++c) {
        const int slot = (int)(c % slots);
        const int64_t r0 = c * chunk_rows;
        const int64_t rows = M - r0 < chunk_rows ? M - r0 : chunk_rows;
        const int64_t rows_pad = pad64(rows);
        uint8_t* q = ring + (size_t)slot * slot_bytes;
        uint8_t* sf = q + (size_t)chunk_rows * (K / 2);
        // pack chunk c into its slot once the GEMM that last read the slot is done
        if (c >= slots && (st = hip_status(hipStreamWaitEvent(rs.pack, rs.consumed[slot], 0))) != NVFP4_OK)
            return st;
        SegParams cs;
        chunk_segments(sp, r0, r0 + rows, &cs);
        const RowGeo g2 = row_geo(rows, rows_pad, K, ldx, kRingPackWgs, 1, 16);
        if ((st = hip_status(launch_modulate_pack(x + r0 * ldx, g2, cs, tensor_scale, q, sf, false, rs.pack))) !=
            NVFP4_OK)
            return st;
        if ((st = hip_status(hipEventRecord(rs.packed[slot], rs.pack))) != NVFP4_OK) return st;
        // the chunk's GEMM on the even or the odd GEMM stream
        const hipStream_t gs = (c & 1) ? rs.gemm_odd : s;
        if ((st = hip_status(hipStreamWaitEvent(gs, rs.packed[slot], 0))) != NVFP4_OK) return st;
        GemmArgs a = ga;
        a.qa = q;
        a.sfa = sf;
        a.out = ga.out + r0 * ga.ldo;
        void* ws = gemm_ws ? gemm_ws + ((c & 1) ? ws_half : 0) : nullptr;
        if ((st = run_gemm(a, rows, rows_pad, ws, ws_half > 0, gs)) != NVFP4_OK) return st;
        if ((st = hip_status(hipEventRecord(rs.consumed[slot], gs))) != NVFP4_OK) return st;
    }
    // the caller's stream continues after the odd GEMMs (whose packs precede them)
    if ((st = hip_status(hipEventRecord(rs.odd_done, rs.gemm_odd))) != NVFP4_OK) return st;
    return hip_status(hipStreamWaitEvent(s, rs.odd_done, 0));
}

size_t nvfp4_ring_slot_bytes(int64_t chunk_rows, int64_t K) {
    if (chunk_rows <= 0 || chunk_rows % 64 != 0 || K <= 0 || K % 64 != 0) return 0;
    return ring_slot_bytes(chunk_rows, K);
}

size_t nvfp4_ring_gemm_workspace_bytes(int64_t M, int64_t chunk_rows, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 64 != 0 || chunk_rows <= 0 || chunk_rows % 64 != 0 ||
        chunk_rows >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31) ||
        gemm_chunk_rows(K) == 0 || chunk_rows > gemm_chunk_rows(K))
        return 0;
    return 2 * ring_gemm_ws_half(M, chunk_rows, N, K);
}

nvfp4_status nvfp4_modulate_gemm_ring(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      const nvfp4_segments* seg, void* workspace, float* tensor_scale,
                                      float* amax_out, uint8_t* ring, int32_t slots, int64_t chunk_rows,
                                      const uint8_t* qw, const uint8_t* sfw, const float* w_scale, int64_t N,
                                      uint16_t* out, int64_t ldo, void* gemm_workspace, size_t gemm_workspace_bytes,
                                      void* stream) {
    nvfp4_status st = check_rows(x, M, K, ldx);
    if (st != NVFP4_OK) return st;
    SegParams sp;
    if ((st = check_segments(seg, M, K, &sp)) != NVFP4_OK) return st;
    if (!workspace || !tensor_scale || !ring) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 4) || !aligned(tensor_scale, 4) || !aligned(amax_out, 4) || !aligned(ring, 16))
        return NVFP4_ERR_ALIGNMENT;
    if (slots < 1 || slots > kMaxRingSlots || chunk_rows <= 0) return NVFP4_ERR_INVALID_ARGUMENT;
    if (chunk_rows % 64 != 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
    // one chunk's packed rows and its GEMM use 32-bit offsets
    if (chunk_rows > gemm_chunk_rows(K) || chunk_rows * (K / 2) >= ((int64_t)1 << 32)) return NVFP4_ERR_SHAPE;
    GemmArgs ga;
    // the activation arguments are per chunk; validate the rest with the first slot
    if ((st = gemm_args(ring, ring + chunk_rows * (K / 2), tensor_scale, chunk_rows < M ? chunk_rows : M,
                        chunk_rows, qw, sfw, w_scale, N, K, out, ldo, &ga)) != NVFP4_OK)
        return st;
    const size_t half = ring_gemm_ws_half(M, chunk_rows, N, K);
    if (half > 0) {
        if (!gemm_workspace || gemm_workspace_bytes < 2 * half) return NVFP4_ERR_INVALID_ARGUMENT;
        if (!aligned(gemm_workspace, 16)) return NVFP4_ERR_ALIGNMENT;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lock(g_ring_mu[dev]);
    RingState* rs = nullptr;
    if ((st = ring_state(dev, &rs)) != NVFP4_OK) return st;
    return ring_run(x, M, K, ldx, sp, workspace, tensor_scale, amax_out, ring, slots, chunk_rows, ga,
                    (uint8_t*)gemm_workspace, half, (hipStream_t)stream, *rs);
}

static nvfp4_status step(int which, const void* a, const void* b, const void* c, void* out, int64_t n,
                         void* stream) {
    if (n < 0 || !out || !a) return NVFP4_ERR_INVALID_ARGUMENT;
    if (n == 0) return NVFP4_OK;
    return hip_status(launch_step(which, a, b, c, out, n, (hipStream_t)stream));
}

nvfp4_status nvfp4_step_modulate(const uint16_t* x, const uint16_t* scale, const uint16_t* shift, uint16_t* y,
                                 int64_t n, void* stream) {
    if (!scale || !shift) return NVFP4_ERR_INVALID_ARGUMENT;
    return step(STEP_MODULATE, x, scale, shift, y, n, stream);
}

nvfp4_status nvfp4_step_swiglu(const uint16_t* g, const uint16_t* u, uint16_t* h, int64_t n, void* stream) {
    if (!u) return NVFP4_ERR_INVALID_ARGUMENT;
    return step(STEP_SWIGLU, g, u, nullptr, h, n, stream);
}

nvfp4_status nvfp4_step_block_scale(const uint16_t* a16, const float* s_g, uint8_t* sf, int64_t n, void* stream) {
    if (!s_g) return NVFP4_ERR_INVALID_ARGUMENT;
    return step(STEP_BLOCK_SCALE, a16, s_g, nullptr, sf, n, stream);
}

nvfp4_status nvfp4_step_element_code(const uint16_t* y, const uint8_t* sf, const float* s_g, uint8_t* code,
                                     int64_t n, void* stream) {
    if (!sf || !s_g) return NVFP4_ERR_INVALID_ARGUMENT;
    return step(STEP_ELEMENT_CODE, y, sf, s_g, code, n, stream);
}

nvfp4_status nvfp4_step_e2m1(const float* v, uint8_t* code, int64_t n, void* stream) {
    return step(STEP_E2M1, v, nullptr, nullptr, code, n, stream);
}

nvfp4_status nvfp4_step_e4m3(const float* t, uint8_t* code, int64_t n, void* stream) {
    return step(STEP_E4M3, t, nullptr, nullptr, code, n, stream);
}

}  // extern "C"
