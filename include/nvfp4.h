/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 activation producer and
 * block-scaled GEMM.
 *
 * What is computed (page title, section):
 *  - "NVFP4 Modulation Producer Fusion", Dataflow / Exactness Contract: the
 *    producer reads the normalized BF16 activation twice, reproduces the
 *    per-segment AdaLN modulation y = (x * (scale + 1)) + shift with BF16
 *    rounding after each operation, reduces |y| to its absolute maximum in the
 *    first pass, and writes packed QDATA and E4M3 block scales into
 *    caller-owned buffers in the second; y never reaches memory.
 *  - "NVFP4 Streaming Design", Numerical Constraint: the tensor's exact BF16
 *    maximum magnitude gives a single FP32 tensor scale; each 16 values get
 *    an E4M3 scale; E2M1 codes come from both scales; no tile can
 *    be packed before the global reduction completes (two passes).
 *  - "FC2 NVFP4 Library Scheduling", Exact Operation: packed activation rows
 *    [M,K] against packed weight rows [N,K], giving BF16 [M,N]; FP32 compute;
 *    alpha = activation tensor scale * weight tensor scale, read from device
 *    memory; no bias; 37,810 logical rows padded to 37,824; the FC2 producer
 *    fuses an exact BF16 SwiGLU.
 *
 * The quantizer the pages leave open is fixed here as:
 *   s_g = amax / 2688 (= 6 * 448), or 1 when amax == 0
 *   sf  = E4M3(RN(RN(a16 / 6) / s_g)), nearest-even, saturating at 448
 *   q   = E2M1(RN(y / RN(float(sf) * s_g))), nearest with ties to the even
 *         code, saturating at +-6, sign kept; all 16 codes 0 when sf is 0
 *         (or the NaN code)
 * with every operation a correctly rounded binary32 operation (no FMA
 * contraction, no flush-to-zero, no approximate reciprocal).
 *
 * Layouts (all row-major, bf16 given as uint16_t bit patterns):
 *   x       [M, D]   bf16, row stride ldx elements
 *   qdata   [M_pad, D/2]  uint8: byte j of a row holds element 2j in bits 3..0
 *                         and element 2j+1 in bits 7..4
 *   sfa     [M_pad, D/16] uint8 E4M3FN, one per 16 consecutive elements
 *   rows M..M_pad-1 of qdata and sfa are written as zero.
 *
 * Conventions:
 *  - Every pointer is device memory except nvfp4_segments.row_start (host).
 *  - Buffers are caller-owned; the library allocates nothing and never
 *    synchronizes the host.  Work is enqueued on `stream` (a hipStream_t
 *    passed as void*; NULL = the null stream) in stream order, so
 *    absmax -> pack -> gemm on one stream need no synchronization.
 *  - Argument errors are reported synchronously, before anything is enqueued.
 *    A launch failure returns NVFP4_ERR_HIP; nvfp4_last_hip_error() gives the
 *    HIP error code of the calling thread's last failure.
 *  - Data-dependent conditions are not reported: a non-finite input yields a
 *    non-finite tensor scale, which the caller can test.
 *  - Calls that share a workspace or outputs must not overlap in time (for
 *    example on two streams without ordering between them).
 *  - The SwiGLU entry points first enqueue a small kernel that fills a
 *    65,536-entry bf16 silu table held in the library's own module-scope
 *    device memory (128 KB per device, part of the code object, not an
 *    allocation); calls overlapping on other streams write identical values.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, ld too small */
    NVFP4_ERR_SHAPE = 2,            /* width not a multiple of 16 (64 for the GEMM's K), M_pad < pad64(M) */
    NVFP4_ERR_ALIGNMENT = 3,        /* base pointer or stride breaks the 16-byte rule */
    NVFP4_ERR_SEGMENTS = 4,         /* bad segment table */
    NVFP4_ERR_HIP = 5               /* kernel launch failed */
} nvfp4_status;

/* Per-segment modulation parameters ("NVFP4 Modulation Producer Fusion",
 * Exactness Contract: each segment selects its own shift and scale).  Segment s
 * covers rows [row_start[s], row_start[s+1]); row_start has count+1 HOST
 * entries with row_start[0] = 0, strictly increasing, row_start[count] = M,
 * 1 <= count <= NVFP4_MAX_SEGMENTS.  shift and scale are DEVICE bf16 arrays
 * [count, D] with row stride ld (>= D, multiple of 8, 16-byte aligned base). */
#define NVFP4_MAX_SEGMENTS 16
typedef struct {
    int32_t count;
    const int64_t* row_start;
    const uint16_t* shift;
    const uint16_t* scale;
    int64_t ld;
} nvfp4_segments;

/* ceil(m / 64) * 64: the padded row count of QDATA/SFA (37,810 -> 37,824,
 * "FC2 NVFP4 Library Scheduling", Exact Operation). */
int64_t nvfp4_padded_rows(int64_t m);

/* Bytes of device workspace the absmax passes and the single launches need
 * (16,640: the global maximum and a counter of the two-pass kernels, and the
 * single launch's result word and one arrival word and one claim word per
 * workgroup).  The workspace must be zero-filled before its first use; after
 * that any sequence of calls may reuse it without clearing (the two-pass
 * kernels return their words to zero, the single launch tags its words with
 * a tag no earlier launch in the process used).  It must not be shared by
 * calls that may overlap. */
size_t nvfp4_absmax_workspace_bytes(void);

/* Byte offset, within that workspace, of a uint32 count of the single
 * launches on it whose grid-barrier wait passed its bound (each such launch
 * adds one, from the device).  The library never resets it; zeroing the
 * workspace does.  A caller checks for timed-out launches without a host
 * synchronization by copying these 4 bytes asynchronously, or by reading them
 * in a later kernel on the same stream.  nvfp4_modulate_quantize_noalloc keeps
 * no such count (it clears its words on every call). */
#define NVFP4_WORKSPACE_TIMEOUT_COUNT_OFFSET 192

/* Sets the bound on the single launches' grid-barrier wait, in microseconds
 * (default 1,000,000), for launches enqueued from then on; returns the
 * previous bound.  A launch whose wait passes the bound completes with a NaN
 * tensor scale and amax, scale code 0x7F and zero codes in every block; 0
 * makes every single launch do so at once (a way to test that path). */
uint64_t nvfp4_set_barrier_timeout_us(uint64_t microseconds);

/* Sets how long a workgroup of a single launch waits at the grid barrier
 * before it computes the pass 1 of workgroups that have not arrived, in
 * microseconds (default 100), for launches enqueued from then on; returns the
 * previous value.  Results do not depend on it; 0 makes every workgroup help
 * from its arrival on (a way to test the helping path). */
uint64_t nvfp4_set_barrier_help_us(uint64_t microseconds);

/* Pass 1 of the modulation producer ("NVFP4 Modulation Producer Fusion",
 * Dataflow, prototype step 1; "NVFP4 Streaming Design", Numerical Constraint,
 * steps 1-2).  Computes y for every element of x [M, D] (row stride ldx, in
 * elements), reduces max |y| over all M rows, and writes
 *   *tensor_scale = amax == 0 ? 1 : RN(amax / 2688)   (device float)
 *   *amax_out     = amax                              (device float, may be NULL)
 * Requirements: M >= 1, D >= 16, D % 16 == 0, ldx >= D, ldx % 8 == 0, x
 * 16-byte aligned; seg valid for M rows and width D. */
nvfp4_status nvfp4_modulate_absmax(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                   const nvfp4_segments* seg, void* workspace,
                                   float* tensor_scale, float* amax_out, void* stream);

/* Pass 2 of the modulation producer ("NVFP4 Modulation Producer Fusion",
 * Dataflow, prototype step 2; "NVFP4 Streaming Design", Numerical Constraint,
 * steps 3-4).  Recomputes y and writes qdata [M_pad, D/2] and sfa
 * [M_pad, D/16] using the device scalar *tensor_scale (normally written by
 * nvfp4_modulate_absmax on the same stream).  Rows M..M_pad-1 are zero.
 * Requirements as for absmax, plus M_pad >= nvfp4_padded_rows(M) and qdata
 * 4-byte aligned. */
nvfp4_status nvfp4_modulate_pack(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                 const nvfp4_segments* seg, const float* tensor_scale,
                                 uint8_t* qdata, uint8_t* sfa, int64_t M_pad, void* stream);

/* Both passes of the modulation producer in one launch (same results as
 * nvfp4_modulate_absmax followed by nvfp4_modulate_pack, byte for byte).  The
 * workgroups (at most as many as the device holds at once) run pass 1, meet
 * at a grid barrier once the global maximum is complete ("NVFP4 Streaming
 * Design", Numerical Constraint: no block is packed before the global
 * reduction, and the two phases may be joined around a grid-wide barrier),
 * and run pass 2, which takes the y of
 * the rows each workgroup visited last from registers and LDS instead of
 * reading x again.  Writes *tensor_scale, *amax_out (may be NULL), qdata and
 * sfa as the two calls do; uses the same workspace.  The barrier needs every
 * workgroup's pass 1, not every workgroup's presence: workgroups that have
 * waited 100 us (nvfp4_set_barrier_help_us) compute the pass 1 of workgroups that could not start (their
 * CUs held by other kernels, for instance another single launch waiting at
 * its own barrier), so concurrent launches complete; the workgroups that
 * start late find the barrier passed.  A wait past the bound of
 * nvfp4_set_barrier_timeout_us (1 s by default) gives a NaN tensor scale and
 * amax, scale code 0x7F and zero codes in every block, for that call only,
 * and adds one to the workspace's timeout count
 * (NVFP4_WORKSPACE_TIMEOUT_COUNT_OFFSET).
 * Calls that can overlap in time must use different workspaces.  Each call
 * takes its barrier tag from the host when it is enqueued, so a call captured
 * into a HIP graph would replay one tag and find the previous replay's words
 * already arrived: under graph capture use nvfp4_modulate_quantize_noalloc
 * (its words are cleared by a kernel on every call) or the two calls
 * nvfp4_modulate_absmax + nvfp4_modulate_pack (whose words return to zero).
 * When D > 16384, or x spans 4 GiB or more, it enqueues the two passes
 * instead.
 * Same requirements as nvfp4_modulate_absmax and nvfp4_modulate_pack
 * together. */
nvfp4_status nvfp4_modulate_quantize(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                     const nvfp4_segments* seg, void* workspace, float* tensor_scale,
                                     float* amax_out, uint8_t* qdata, uint8_t* sfa, int64_t M_pad,
                                     void* stream);

/* nvfp4_modulate_quantize for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same results, byte for byte, with no workspace argument.
 * The grid barrier's words live in a fixed 16,640-byte array inside the
 * library's code object, one copy per device (held until the process ends);
 * every shape nvfp4_modulate_quantize accepts fits it.  The call enqueues a
 * small kernel that zeroes those words, then the producer, on `stream`; it
 * calls no allocator.  Because the words are cleared by a kernel, a call
 * captured into a graph replays correctly (make one call outside capture
 * first: it looks up the array's address and the grid size).  All calls on one device share the array: calls that
 * can overlap in time on one device (two streams without ordering between
 * them) race and must not be made.  Same arguments, requirements and errors
 * as nvfp4_modulate_quantize, without the workspace. */
nvfp4_status nvfp4_modulate_quantize_noalloc(const uint16_t* x, int64_t M, int64_t D, int64_t ldx,
                                             const nvfp4_segments* seg, float* tensor_scale, float* amax_out,
                                             uint8_t* qdata, uint8_t* sfa, int64_t M_pad, void* stream);

/* The plain quantizer: nvfp4_modulate_quantize with y = x (no modulation), for
 * activations that need none (the attention-output projection's input,
 * "NVFP4 Streaming Design", P0/P2: the widths 5376, 7168, 14336) and for
 * prepacking weights.  Same launch structure, outputs, workspace,
 * requirements and graph-capture caveat, without the segment table. */
nvfp4_status nvfp4_quantize(const uint16_t* x, int64_t M, int64_t D, int64_t ldx, void* workspace,
                            float* tensor_scale, float* amax_out, uint8_t* qdata, uint8_t* sfa, int64_t M_pad,
                            void* stream);

/* Pass 1 of the SwiGLU producer ("FC2 NVFP4 Library Scheduling", Exact
 * Operation and Current Baseline: exact BF16 SwiGLU fused into NVFP4
 * production).  h = bf16(bf16(silu(g)) * u) with silu(g) = g / (1 + exp(-g))
 * in binary32 with a correctly rounded exp; g = gate[r*ld + c],
 * u = up[r*ld + c] for c < F.  For one [M, 2F] gate/up tensor pass
 * gate = GU, up = GU + F, ld = 2F.  Writes tensor scale and amax as
 * nvfp4_modulate_absmax.  Requirements: F % 16 == 0, ld >= F, ld % 8 == 0,
 * gate and up 16-byte aligned. */
nvfp4_status nvfp4_swiglu_absmax(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F,
                                 int64_t ld, void* workspace, float* tensor_scale, float* amax_out,
                                 void* stream);

/* Pass 2 of the SwiGLU producer: recomputes h and writes qdata [M_pad, F/2]
 * and sfa [M_pad, F/16] with the device *tensor_scale; pad rows zero. */
nvfp4_status nvfp4_swiglu_pack(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F,
                               int64_t ld, const float* tensor_scale, uint8_t* qdata, uint8_t* sfa,
                               int64_t M_pad, void* stream);

/* Both SwiGLU passes in one call (same results as nvfp4_swiglu_absmax
 * followed by nvfp4_swiglu_pack, byte for byte): after the silu table fill,
 * one launch runs pass 1, a grid barrier and pass 2, keeping h of the rows
 * each workgroup visited last in registers, as nvfp4_modulate_quantize does
 * (same workspace, the same barrier with helping, the same bound, and the
 * same caveat under graph capture: use the two calls there).  When
 * F > 16384, or gate/up spans
 * 4 GiB or more, it enqueues the two passes instead.  Same arguments,
 * requirements and errors as the two calls together. */
nvfp4_status nvfp4_swiglu_quantize(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t F,
                                   int64_t ld, void* workspace, float* tensor_scale, float* amax_out,
                                   uint8_t* qdata, uint8_t* sfa, int64_t M_pad, void* stream);

/* Block-scaled GEMM ("FC2 NVFP4 Library Scheduling", Exact Operation;
 * "NVFP4 Streaming Design", P0: FP32 global-scale product applied before the
 * BF16 conversion):
 *   out[m][n] = bf16(RN(alpha * sum_k A[m][k] * W[n][k])),  m < M, n < N
 *   A = e2m1(qa) * e4m3(sfa), W = e2m1(qw) * e4m3(sfw),
 *   alpha = RN(*a_scale * *w_scale)  (both device floats)
 * qa [M_pad, K/2], sfa [M_pad, K/16] (rows >= M are read as padding and
 * ignored), qw [N, K/2], sfw [N, K/16], out [M, ldo] bf16.  The K sum is
 * accumulated in binary32 in an order of the kernel's choosing.
 * Requirements: K % 64 == 0, N % 16 == 0, ldo >= N, ldo % 4 == 0,
 * M_pad >= M, qa/qw 16-byte aligned, sfa/sfw 4-byte aligned, out 8-byte
 * aligned; N * K/2 < 2^32 (the packed weight under 4 GiB), K <= 2^25,
 * M_pad < 2^31.  The activation may exceed 4 GiB: the rows are then computed
 * in chunks of floor((2^32 - 1) / (K/2)) rounded down to a multiple of 256, one
 * launch sequence per chunk in stream order. */
nvfp4_status nvfp4_gemm(const uint8_t* qa, const uint8_t* sfa, const float* a_scale, int64_t M,
                        int64_t M_pad, const uint8_t* qw, const uint8_t* sfw, const float* w_scale,
                        int64_t N, int64_t K, uint16_t* out, int64_t ldo, void* stream);

/* Bytes of device workspace nvfp4_gemm_ws uses for an [M,K] x [N,K] product
 * (0 when it has nothing to split; for an activation in several row chunks,
 * the largest chunk's need).  Depends on the shape only. */
size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* nvfp4_gemm with a caller-owned workspace of at least
 * nvfp4_gemm_workspace_bytes(M, N, K) bytes (16-byte aligned; may be NULL when
 * that is 0).  The output tiles are computed in waves of 256 workgroups; when
 * the last wave would fill at most a third of the chip, its tiles are each
 * computed as several K ranges by separate workgroups whose binary32 partial
 * sums land in the workspace, then added in K order and scaled by alpha.  The
 * result satisfies the same contract as nvfp4_gemm (only the binary32
 * summation order differs).  The workspace holds no state between calls;
 * calls sharing it must not overlap.  Like nvfp4_gemm it enqueues kernels
 * only (no memset, no allocation), so a call can be captured into a HIP graph
 * and replayed with new operands in the same buffers.  Same requirements and errors as
 * nvfp4_gemm, plus NVFP4_ERR_INVALID_ARGUMENT for a missing or short
 * workspace. */
nvfp4_status nvfp4_gemm_ws(const uint8_t* qa, const uint8_t* sfa, const float* a_scale, int64_t M,
                           int64_t M_pad, const uint8_t* qw, const uint8_t* sfw, const float* w_scale,
                           int64_t N, int64_t K, uint16_t* out, int64_t ldo, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Per-segment gates of the residual epilogue: segment s covers output rows
 * [row_start[s], row_start[s+1]) (count+1 HOST entries, 0 .. M, strictly
 * increasing, 1 <= count <= NVFP4_MAX_SEGMENTS) and uses the DEVICE bf16 gate
 * row gate[s * ld .. s * ld + N). */
typedef struct {
    int32_t count;
    const int64_t* row_start;
    const uint16_t* gate;
    int64_t ld;
} nvfp4_row_gates;

/* nvfp4_gemm_ws followed by the exact residual epilogue ("NVFP4 Streaming
 * Design", P4: the GEMM result rounded to BF16, scaled by the gate, added to
 * the residual and rounded to BF16 again), fused into the GEMM's store:
 *   o   = bf16(RN(alpha * sum_k A[m][k] * W[n][k]))   (the nvfp4_gemm output)
 *   out = bf16(RN(residual[m][n] + bf16(RN(gate[s][n] * o))))
 * with s the segment of row m; residual is bf16 [M, ldr].  out may be the
 * residual itself (same pointer and stride: each element is read before it is
 * written, by the same thread); otherwise the two must not overlap.  Same
 * requirements and workspace as nvfp4_gemm_ws, plus: gate and residual 8-byte
 * aligned, gates->ld and ldr >= N and multiples of 4; a bad gate table returns
 * NVFP4_ERR_SEGMENTS. */
nvfp4_status nvfp4_gemm_gate_residual(const uint8_t* qa, const uint8_t* sfa, const float* a_scale, int64_t M,
                                      int64_t M_pad, const uint8_t* qw, const uint8_t* sfw, const float* w_scale,
                                      int64_t N, int64_t K, const nvfp4_row_gates* gates, const uint16_t* residual,
                                      int64_t ldr, uint16_t* out, int64_t ldo, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ---- Packed-tile ring ---------------------------------------------------
 * "NVFP4 Streaming Design", P2 (N-group reuse): instead of materializing the
 * whole packed activation, a bounded ring of packed row slots; one tensor
 * scale from the full activation is reused by every chunk, each chunk of rows
 * is packed into a slot and multiplied by the whole weight, and the slot is
 * recycled.  The pages chose 2048-row chunks (18 full ones and a last one of
 * 946 rows at 37,810 rows) and reported the ring slower than the
 * materialized path at block level on their GPU; here it is an opt-in entry
 * point with the same results as nvfp4_modulate_quantize followed by
 * nvfp4_gemm_ws, so the two can be compared. */

/* Bytes of one ring slot: chunk_rows rows of QDATA (K/2 bytes each) followed
 * by chunk_rows rows of SFA (K/16 bytes each).  0 for an invalid argument
 * (chunk_rows and K must be positive multiples of 64). */
size_t nvfp4_ring_slot_bytes(int64_t chunk_rows, int64_t K);

/* Bytes of GEMM workspace nvfp4_modulate_gemm_ring needs: two K-split
 * workspaces (one per GEMM stream) for the larger of a full and the last
 * chunk.  0 when no chunk's GEMM splits (or for an invalid argument). */
size_t nvfp4_ring_gemm_workspace_bytes(int64_t M, int64_t chunk_rows, int64_t N, int64_t K);

/* Modulation producer and GEMM through a ring of `slots` packed slots:
 *   1. pass 1 over all M rows of x [M, K]: *tensor_scale, *amax_out (may be
 *      NULL), as nvfp4_modulate_absmax (same workspace rules);
 *   2. for chunk c (rows [c*chunk_rows, min(M, (c+1)*chunk_rows))): pass 2 of
 *      its rows into slot c % slots (rows past the chunk's last row up to the
 *      next multiple of 64 are zero), then the GEMM of that slot against the
 *      packed weight qw [N, K/2], sfw [N, K/16] with alpha = RN(*tensor_scale
 *      * *w_scale), written to out rows [c*chunk_rows, ...) (bf16 [M, ldo]).
 * The slot bytes of chunk c equal rows c*chunk_rows .. of the QDATA/SFA that
 * nvfp4_modulate_quantize writes; the outputs satisfy nvfp4_gemm's contract
 * and, when chunk_rows is a multiple of 256, equal nvfp4_gemm_ws's bit for bit
 * except in tiles that either call computes as K-split pieces.
 * Streams: pass 1 and the even chunks' GEMMs run on `stream`; the packs and
 * the odd chunks' GEMMs on two streams the library creates once per device
 * (default priority), ordered by events: a pack waits for the GEMM that last
 * read its slot, a GEMM for its chunk's pack, and `stream` waits for all of it
 * before its next work, so the call is stream-ordered for the caller.  No
 * workgroup waits on another.  The ring (16-byte aligned, at least
 * slots * nvfp4_ring_slot_bytes(chunk_rows, K) bytes) and gemm_workspace
 * (nvfp4_ring_gemm_workspace_bytes) are caller-owned and must not be shared
 * with calls that may overlap; calls on one device are enqueued one at a time
 * (a host lock).
 * Requirements: those of nvfp4_modulate_absmax, nvfp4_modulate_pack and
 * nvfp4_gemm_ws; 1 <= slots <= 64; chunk_rows a multiple of 64 with
 * chunk_rows * K/2 < 2^32. */
nvfp4_status nvfp4_modulate_gemm_ring(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      const nvfp4_segments* seg, void* workspace, float* tensor_scale,
                                      float* amax_out, uint8_t* ring, int32_t slots, int64_t chunk_rows,
                                      const uint8_t* qw, const uint8_t* sfw, const float* w_scale, int64_t N,
                                      uint16_t* out, int64_t ldo, void* gemm_workspace, size_t gemm_workspace_bytes,
                                      void* stream);

/* ---- Single-step entry points ------------------------------------------
 * Elementwise versions of single producer steps, running the very device
 * functions the producer kernels use, so that each step can be checked over
 * its whole input domain.  All arrays are device memory of n elements. */

/* a1: y[i] = bf16(bf16(bf16(x*bf16(scale+1))) + shift)
 * ("NVFP4 Modulation Producer Fusion", Exactness Contract). */
nvfp4_status nvfp4_step_modulate(const uint16_t* x, const uint16_t* scale, const uint16_t* shift,
                                 uint16_t* y, int64_t n, void* stream);
/* a6: h[i] = bf16(bf16(silu(g)) * u) ("FC2 NVFP4 Library Scheduling"). */
nvfp4_status nvfp4_step_swiglu(const uint16_t* g, const uint16_t* u, uint16_t* h, int64_t n,
                               void* stream);
/* a3: sf[i] = E4M3(RN(RN(a16[i] / 6) / *s_g)) with a16 given as bf16 bits
 * ("NVFP4 Streaming Design", Numerical Constraint, step 3). */
nvfp4_status nvfp4_step_block_scale(const uint16_t* a16, const float* s_g, uint8_t* sf, int64_t n,
                                    void* stream);
/* a4: code[i] = E2M1(RN(y[i] / RN(float(sf[i]) * *s_g))), 0 when sf[i] is 0
 * or the NaN code ("NVFP4 Streaming Design", Numerical Constraint, step 4). */
nvfp4_status nvfp4_step_element_code(const uint16_t* y, const uint8_t* sf, const float* s_g,
                                     uint8_t* code, int64_t n, void* stream);
/* E2M1 encoding of binary32 values (the conversion behind a4):
 * code[i] = E2M1(v[i]) with ties to the even code and saturation at +-6. */
nvfp4_status nvfp4_step_e2m1(const float* v, uint8_t* code, int64_t n, void* stream);
/* E4M3 encoding of non-negative binary32 values (the conversion behind a3). */
nvfp4_status nvfp4_step_e4m3(const float* t, uint8_t* code, int64_t n, void* stream);

const char* nvfp4_status_string(nvfp4_status s);
int nvfp4_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
