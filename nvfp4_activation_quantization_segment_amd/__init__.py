"""Python binding of the MI355X NVFP4 activation producer and block-scaled GEMM.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libnvfp4.so`` (built in-tree by ``build.py``).  PyTorch provides device
memory and the current stream.  There is no fallback: importing this package
without the built library raises.

Functions named like the C entry points (``nvfp4_modulate_absmax`` ...) take
torch tensors and the same arguments as the C ABI (``include/nvfp4.h``);
``modulate_quantize``, ``swiglu_quantize`` and ``gemm`` are conveniences that
allocate their outputs with torch.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that the library must share

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK = 0
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "misaligned pointer or stride",
           4: "invalid segment table", 5: "HIP launch failure"}
MAX_SEGMENTS = 16


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        msg = f"{fn}: {_STATUS.get(status, status)}"
        if status == 5:
            msg += f" (hip error {hip_error})"
        super().__init__(msg)
        self.status = status


class Segments(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("row_start", ctypes.POINTER(ctypes.c_int64)),
                ("shift", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("ld", ctypes.c_int64)]


class RowGates(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("row_start", ctypes.POINTER(ctypes.c_int64)),
                ("gate", ctypes.c_void_p), ("ld", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run nvfp4_activation_quantization_segment_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, V = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    SEG = ctypes.POINTER(Segments)
    GATES = ctypes.POINTER(RowGates)
    sigs = {
        "nvfp4_padded_rows": (I64, [I64]),
        "nvfp4_absmax_workspace_bytes": (ctypes.c_size_t, []),
        "nvfp4_set_barrier_timeout_us": (ctypes.c_uint64, [ctypes.c_uint64]),
        "nvfp4_set_barrier_help_us": (ctypes.c_uint64, [ctypes.c_uint64]),
        "nvfp4_modulate_absmax": (I32, [P, I64, I64, I64, SEG, P, P, P, V]),
        "nvfp4_modulate_pack": (I32, [P, I64, I64, I64, SEG, P, P, P, I64, V]),
        "nvfp4_modulate_quantize": (I32, [P, I64, I64, I64, SEG, P, P, P, P, P, I64, V]),
        "nvfp4_modulate_quantize_noalloc": (I32, [P, I64, I64, I64, SEG, P, P, P, P, I64, V]),
        "nvfp4_quantize": (I32, [P, I64, I64, I64, P, P, P, P, P, I64, V]),
        "nvfp4_swiglu_absmax": (I32, [P, P, I64, I64, I64, P, P, P, V]),
        "nvfp4_swiglu_pack": (I32, [P, P, I64, I64, I64, P, P, P, I64, V]),
        "nvfp4_swiglu_quantize": (I32, [P, P, I64, I64, I64, P, P, P, P, P, I64, V]),
        "nvfp4_gemm": (I32, [P, P, P, I64, I64, P, P, P, I64, I64, P, I64, V]),
        "nvfp4_gemm_workspace_bytes": (ctypes.c_size_t, [I64, I64, I64]),
        "nvfp4_gemm_ws": (I32, [P, P, P, I64, I64, P, P, P, I64, I64, P, I64, P, ctypes.c_size_t, V]),
        "nvfp4_gemm_gate_residual": (I32, [P, P, P, I64, I64, P, P, P, I64, I64, GATES, P, I64, P, I64, P,
                                            ctypes.c_size_t, V]),
        "nvfp4_ring_slot_bytes": (ctypes.c_size_t, [I64, I64]),
        "nvfp4_ring_gemm_workspace_bytes": (ctypes.c_size_t, [I64, I64, I64, I64]),
        "nvfp4_modulate_gemm_ring": (I32, [P, I64, I64, I64, SEG, P, P, P, P, I32, I64, P, P, P, I64, P, I64, P,
                                           ctypes.c_size_t, V]),
        "nvfp4_step_modulate": (I32, [P, P, P, P, I64, V]),
        "nvfp4_step_swiglu": (I32, [P, P, P, I64, V]),
        "nvfp4_step_block_scale": (I32, [P, P, P, I64, V]),
        "nvfp4_step_element_code": (I32, [P, P, P, P, I64, V]),
        "nvfp4_step_e2m1": (I32, [P, P, I64, V]),
        "nvfp4_step_e4m3": (I32, [P, P, I64, V]),
        "nvfp4_status_string": (ctypes.c_char_p, [I32]),
        "nvfp4_last_hip_error": (ctypes.c_int, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t) -> ctypes.c_void_p | None:
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(fn: str, status: int):
    if status != NVFP4_OK:
        raise Nvfp4Error(fn, status, lib.nvfp4_last_hip_error())


def _bits16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected bf16 (or its 16-bit pattern), got {t.dtype}")
    return t


def make_segments(row_start, shift: torch.Tensor, scale: torch.Tensor):
    """Build the C segment table; returns (struct, keepalive)."""
    rs = (ctypes.c_int64 * len(row_start))(*[int(r) for r in row_start])
    _bits16(shift)
    _bits16(scale)
    if shift.shape != scale.shape or shift.dim() != 2 or shift.stride(1) != 1 or scale.stride(0) != shift.stride(0):
        raise ValueError("shift/scale must be [S, D] with unit column stride and equal row strides")
    seg = Segments(len(row_start) - 1, ctypes.cast(rs, ctypes.POINTER(ctypes.c_int64)), shift.data_ptr(),
                   scale.data_ptr(), shift.stride(0))
    return seg, (rs, shift, scale)


_workspaces: dict[tuple[int, int], torch.Tensor] = {}


def _torch_stream(stream, dev: torch.device):
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=dev)


def _capturing(st) -> bool:
    """Whether work enqueued on torch stream st is being captured into a graph."""
    with torch.cuda.stream(st):
        return torch.cuda.is_current_stream_capturing()


def workspace(device=None, stream=None) -> torch.Tensor:
    """The producers' workspace for one (device, stream) pair, zero-filled on
    that stream when first made.  Calls on one stream run in order and may
    share a workspace; calls that may overlap must not (their maxima and
    barrier words would mix), so every stream gets its own."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    ts = _torch_stream(stream, dev)
    key = (dev.index, int(ts.cuda_stream))
    ws = _workspaces.get(key)
    if ws is None:
        with torch.cuda.stream(ts):
            ws = torch.zeros(int(lib.nvfp4_absmax_workspace_bytes()), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


WORKSPACE_TIMEOUT_COUNT_OFFSET = 192  # NVFP4_WORKSPACE_TIMEOUT_COUNT_OFFSET


def workspace_timeouts(ws: torch.Tensor) -> int:
    """The workspace's count of single launches whose grid-barrier wait passed
    its bound (synchronizes with the workspace's stream to read it; a caller
    that must not synchronize copies the 4 bytes asynchronously instead)."""
    o = WORKSPACE_TIMEOUT_COUNT_OFFSET
    return int(ws[o:o + 4].view(torch.int32).item())


def set_barrier_timeout_us(microseconds: int) -> int:
    """Bound on the single launches' grid-barrier wait (default 1 s); returns
    the previous bound.  0 makes every single launch give up at once."""
    return int(lib.nvfp4_set_barrier_timeout_us(int(microseconds)))


def set_barrier_help_us(microseconds: int) -> int:
    """Wait at the grid barrier before a workgroup computes absent workgroups'
    pass 1 (default 100 us); returns the previous value.  0: help at once."""
    return int(lib.nvfp4_set_barrier_help_us(int(microseconds)))


def padded_rows(m: int) -> int:
    return int(lib.nvfp4_padded_rows(int(m)))


# ---------------------------------------------------------------------------
# C entry points, same names and arguments
# ---------------------------------------------------------------------------
def nvfp4_modulate_absmax(x, M, D, ldx, seg, ws, tensor_scale, amax_out=None, stream=None):
    _check("nvfp4_modulate_absmax",
           lib.nvfp4_modulate_absmax(_ptr(x), M, D, ldx, ctypes.byref(seg), _ptr(ws), _ptr(tensor_scale),
                                     _ptr(amax_out), _stream(stream)))


def nvfp4_modulate_pack(x, M, D, ldx, seg, tensor_scale, qdata, sfa, M_pad, stream=None):
    _check("nvfp4_modulate_pack",
           lib.nvfp4_modulate_pack(_ptr(x), M, D, ldx, ctypes.byref(seg), _ptr(tensor_scale), _ptr(qdata),
                                   _ptr(sfa), M_pad, _stream(stream)))


def nvfp4_modulate_quantize(x, M, D, ldx, seg, ws, tensor_scale, amax_out, qdata, sfa, M_pad, stream=None):
    _check("nvfp4_modulate_quantize",
           lib.nvfp4_modulate_quantize(_ptr(x), M, D, ldx, ctypes.byref(seg), _ptr(ws), _ptr(tensor_scale),
                                       _ptr(amax_out), _ptr(qdata), _ptr(sfa), M_pad, _stream(stream)))


def nvfp4_modulate_quantize_noalloc(x, M, D, ldx, seg, tensor_scale, amax_out, qdata, sfa, M_pad, stream=None):
    _check("nvfp4_modulate_quantize_noalloc",
           lib.nvfp4_modulate_quantize_noalloc(_ptr(x), M, D, ldx, ctypes.byref(seg), _ptr(tensor_scale),
                                               _ptr(amax_out), _ptr(qdata), _ptr(sfa), M_pad, _stream(stream)))


def nvfp4_quantize(x, M, D, ldx, ws, tensor_scale, amax_out, qdata, sfa, M_pad, stream=None):
    _check("nvfp4_quantize",
           lib.nvfp4_quantize(_ptr(x), M, D, ldx, _ptr(ws), _ptr(tensor_scale), _ptr(amax_out), _ptr(qdata), _ptr(sfa),
                              M_pad, _stream(stream)))


def nvfp4_swiglu_absmax(gate, up, M, F, ld, ws, tensor_scale, amax_out=None, stream=None):
    _check("nvfp4_swiglu_absmax",
           lib.nvfp4_swiglu_absmax(_ptr(gate), _ptr(up), M, F, ld, _ptr(ws), _ptr(tensor_scale), _ptr(amax_out),
                                   _stream(stream)))


def nvfp4_swiglu_pack(gate, up, M, F, ld, tensor_scale, qdata, sfa, M_pad, stream=None):
    _check("nvfp4_swiglu_pack",
           lib.nvfp4_swiglu_pack(_ptr(gate), _ptr(up), M, F, ld, _ptr(tensor_scale), _ptr(qdata), _ptr(sfa), M_pad,
                                 _stream(stream)))


def nvfp4_swiglu_quantize(gate, up, M, F, ld, workspace, tensor_scale, amax, qdata, sfa, M_pad, stream=None):
    _check("nvfp4_swiglu_quantize",
           lib.nvfp4_swiglu_quantize(_ptr(gate), _ptr(up), M, F, ld, _ptr(workspace), _ptr(tensor_scale), _ptr(amax),
                                     _ptr(qdata), _ptr(sfa), M_pad, _stream(stream)))


def nvfp4_gemm(qa, sfa, a_scale, M, M_pad, qw, sfw, w_scale, N, K, out, ldo, stream=None):
    _check("nvfp4_gemm",
           lib.nvfp4_gemm(_ptr(qa), _ptr(sfa), _ptr(a_scale), M, M_pad, _ptr(qw), _ptr(sfw), _ptr(w_scale), N, K,
                          _ptr(out), ldo, _stream(stream)))


def nvfp4_gemm_workspace_bytes(M, N, K):
    return int(lib.nvfp4_gemm_workspace_bytes(M, N, K))


def nvfp4_gemm_ws(qa, sfa, a_scale, M, M_pad, qw, sfw, w_scale, N, K, out, ldo, workspace, workspace_bytes,
                  stream=None):
    _check("nvfp4_gemm_ws",
           lib.nvfp4_gemm_ws(_ptr(qa), _ptr(sfa), _ptr(a_scale), M, M_pad, _ptr(qw), _ptr(sfw), _ptr(w_scale), N, K,
                             _ptr(out), ldo, _ptr(workspace), workspace_bytes, _stream(stream)))


def make_row_gates(row_start, gate: torch.Tensor):
    """Build the C gate table; returns (struct, keepalive)."""
    rs = (ctypes.c_int64 * len(row_start))(*[int(r) for r in row_start])
    _bits16(gate)
    if gate.dim() != 2 or gate.stride(1) != 1:
        raise ValueError("gate must be [S, N] with unit column stride")
    g = RowGates(len(row_start) - 1, ctypes.cast(rs, ctypes.POINTER(ctypes.c_int64)), gate.data_ptr(), gate.stride(0))
    return g, (rs, gate)


def nvfp4_gemm_gate_residual(qa, sfa, a_scale, M, M_pad, qw, sfw, w_scale, N, K, gates, residual, ldr, out, ldo,
                             workspace, workspace_bytes, stream=None):
    _check("nvfp4_gemm_gate_residual",
           lib.nvfp4_gemm_gate_residual(_ptr(qa), _ptr(sfa), _ptr(a_scale), M, M_pad, _ptr(qw), _ptr(sfw),
                                        _ptr(w_scale), N, K, ctypes.byref(gates), _ptr(residual), ldr, _ptr(out), ldo,
                                        _ptr(workspace), workspace_bytes, _stream(stream)))


def nvfp4_ring_slot_bytes(chunk_rows, K):
    return int(lib.nvfp4_ring_slot_bytes(chunk_rows, K))


def nvfp4_ring_gemm_workspace_bytes(M, chunk_rows, N, K):
    return int(lib.nvfp4_ring_gemm_workspace_bytes(M, chunk_rows, N, K))


def nvfp4_modulate_gemm_ring(x, M, K, ldx, seg, ws, tensor_scale, amax_out, ring, slots, chunk_rows, qw, sfw,
                             w_scale, N, out, ldo, gemm_workspace, gemm_workspace_bytes, stream=None):
    _check("nvfp4_modulate_gemm_ring",
           lib.nvfp4_modulate_gemm_ring(_ptr(x), M, K, ldx, ctypes.byref(seg), _ptr(ws), _ptr(tensor_scale),
                                        _ptr(amax_out), _ptr(ring), slots, chunk_rows, _ptr(qw), _ptr(sfw),
                                        _ptr(w_scale), N, _ptr(out), ldo, _ptr(gemm_workspace),
                                        gemm_workspace_bytes, _stream(stream)))


def nvfp4_step_modulate(x, scale, shift, y, n, stream=None):
    _check("nvfp4_step_modulate",
           lib.nvfp4_step_modulate(_ptr(x), _ptr(scale), _ptr(shift), _ptr(y), n, _stream(stream)))


def nvfp4_step_swiglu(g, u, h, n, stream=None):
    _check("nvfp4_step_swiglu", lib.nvfp4_step_swiglu(_ptr(g), _ptr(u), _ptr(h), n, _stream(stream)))


def nvfp4_step_block_scale(a16, s_g, sf, n, stream=None):
    _check("nvfp4_step_block_scale", lib.nvfp4_step_block_scale(_ptr(a16), _ptr(s_g), _ptr(sf), n, _stream(stream)))


def nvfp4_step_element_code(y, sf, s_g, code, n, stream=None):
    _check("nvfp4_step_element_code",
           lib.nvfp4_step_element_code(_ptr(y), _ptr(sf), _ptr(s_g), _ptr(code), n, _stream(stream)))


def nvfp4_step_e2m1(v, code, n, stream=None):
    _check("nvfp4_step_e2m1", lib.nvfp4_step_e2m1(_ptr(v), _ptr(code), n, _stream(stream)))


def nvfp4_step_e4m3(t, code, n, stream=None):
    _check("nvfp4_step_e4m3", lib.nvfp4_step_e4m3(_ptr(t), _ptr(code), n, _stream(stream)))


# ---------------------------------------------------------------------------
# conveniences (torch allocates the outputs)
# ---------------------------------------------------------------------------
def modulate_quantize(x: torch.Tensor, row_start, shift: torch.Tensor, scale: torch.Tensor, m_pad: int | None = None,
                      stream=None, single_pass: bool = True):
    """x [M, D] bf16 -> (qdata [M_pad, D/2] u8, sfa [M_pad, D/16] u8, tensor_scale f32[1], amax f32[1]).

    single_pass: one nvfp4_modulate_quantize launch; else nvfp4_modulate_absmax
    then nvfp4_modulate_pack (identical bytes).  Under graph capture the two
    launches are used either way: the single launch's barrier tag comes from
    the host when it is enqueued, so a replay would meet the previous replay's
    words, while the two-pass words return to zero after every call."""
    _bits16(x)
    M, D = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    m_pad = padded_rows(M) if m_pad is None else m_pad
    seg, keep = make_segments(row_start, shift, scale)
    dev = x.device
    st = _torch_stream(stream, dev)
    with torch.cuda.stream(st):  # outputs belong to the stream that writes them
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        amax = torch.empty(1, dtype=torch.float32, device=dev)
        q = torch.empty((m_pad, D // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((m_pad, D // 16), dtype=torch.uint8, device=dev)
    if single_pass and not _capturing(st):
        nvfp4_modulate_quantize(x, M, D, x.stride(0), seg, workspace(dev, st), ts, amax, q, s, m_pad, st)
    else:
        nvfp4_modulate_absmax(x, M, D, x.stride(0), seg, workspace(dev, st), ts, amax, st)
        nvfp4_modulate_pack(x, M, D, x.stride(0), seg, ts, q, s, m_pad, st)
    del keep
    return q, s, ts, amax


def swiglu_quantize(gu: torch.Tensor, m_pad: int | None = None, stream=None, combined: bool = True):
    """gate/up [M, 2F] bf16 (gate = first F columns) -> (qdata, sfa, tensor_scale, amax).

    combined: one nvfp4_swiglu_quantize call; else nvfp4_swiglu_absmax then
    nvfp4_swiglu_pack (identical bytes); the latter under graph capture, as in
    modulate_quantize."""
    _bits16(gu)
    M, F2 = gu.shape
    F = F2 // 2
    if gu.stride(1) != 1:
        raise ValueError("gate/up must have unit column stride")
    m_pad = padded_rows(M) if m_pad is None else m_pad
    dev = gu.device
    st = _torch_stream(stream, dev)
    with torch.cuda.stream(st):
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        amax = torch.empty(1, dtype=torch.float32, device=dev)
        q = torch.empty((m_pad, F // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((m_pad, F // 16), dtype=torch.uint8, device=dev)
    up = gu.data_ptr() + F * gu.element_size()
    if combined and not _capturing(st):
        nvfp4_swiglu_quantize(gu, up, M, F, gu.stride(0), workspace(dev, st), ts, amax, q, s, m_pad, st)
    else:
        nvfp4_swiglu_absmax(gu, up, M, F, gu.stride(0), workspace(dev, st), ts, amax, st)
        nvfp4_swiglu_pack(gu, up, M, F, gu.stride(0), ts, q, s, m_pad, st)
    return q, s, ts, amax


_identity: dict[tuple[int, int], tuple[torch.Tensor, torch.Tensor]] = {}


def _identity_modulation(dev: torch.device, D: int, st):
    """shift = -0 and scale = +0 rows of width D (y = bf16(bf16(x * 1) + -0) = x
    for every bf16 x), kept for the life of the process: a graph that captured
    a call reads them on every replay."""
    key = (dev.index, D)
    if key not in _identity:
        with torch.cuda.stream(st):
            _identity[key] = (torch.full((1, D), -0.0, dtype=torch.bfloat16, device=dev),
                              torch.zeros((1, D), dtype=torch.bfloat16, device=dev))
    return _identity[key]


def quantize(x: torch.Tensor, m_pad: int | None = None, stream=None):
    """Plain quantizer: x [M, D] bf16 -> (qdata [M_pad, D/2], sfa [M_pad, D/16], tensor_scale f32[1], amax f32[1]).

    Under graph capture (see modulate_quantize) it runs the two modulation
    passes with the identity modulation, scale +0 and shift -0, which leaves
    every bf16 value as it is: the same bytes."""
    _bits16(x)
    M, D = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    m_pad = padded_rows(M) if m_pad is None else m_pad
    dev = x.device
    st = _torch_stream(stream, dev)
    with torch.cuda.stream(st):
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        amax = torch.empty(1, dtype=torch.float32, device=dev)
        q = torch.empty((m_pad, D // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((m_pad, D // 16), dtype=torch.uint8, device=dev)
    if _capturing(st):
        shift0, scale0 = _identity_modulation(dev, D, st)
        seg, keep = make_segments([0, M], shift0, scale0)
        nvfp4_modulate_absmax(x, M, D, x.stride(0), seg, workspace(dev, st), ts, amax, st)
        nvfp4_modulate_pack(x, M, D, x.stride(0), seg, ts, q, s, m_pad, st)
        del keep
    else:
        nvfp4_quantize(x, M, D, x.stride(0), workspace(dev, st), ts, amax, q, s, m_pad, st)
    return q, s, ts, amax


def quantize_weight(w: torch.Tensor, stream=None):
    """Prepack a bf16 weight [N, K] to NVFP4 with the plain quantizer: returns
    (qw [N, K/2], sfw [N, K/16], w_scale f32[1])."""
    N, K = w.shape
    q, s, ts, _ = quantize(w, stream=stream)
    return q[:N], s[:N], ts


def gemm(qa, sfa, a_scale, M: int, qw, sfw, w_scale, out: torch.Tensor | None = None, stream=None,
         workspace: torch.Tensor | None = None):
    """out [M, N] bf16 = bf16(a_scale * w_scale * dequant(qa) dequant(qw)^T).

    Runs nvfp4_gemm_ws on `stream` (default: the current stream); a workspace
    of nvfp4_gemm_workspace_bytes(M, N, K) bytes is allocated with torch when
    none is given.  The output and that workspace are allocated on the stream
    the GEMM runs on, so the caching allocator hands the workspace to no other
    stream's allocation before the GEMM has finished with it."""
    M_pad, Kh = qa.shape
    N = qw.shape[0]
    K = 2 * Kh
    st = _torch_stream(stream, qa.device)
    need = nvfp4_gemm_workspace_bytes(M, N, K)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=qa.device)
    nvfp4_gemm_ws(qa, sfa, a_scale, M, M_pad, qw, sfw, w_scale, N, K, out, out.stride(0), workspace,
                  need, st)
    return out


def modulate_gemm_ring(x: torch.Tensor, row_start, shift: torch.Tensor, scale: torch.Tensor, qw, sfw, w_scale,
                       chunk_rows: int = 2048, slots: int = 2, out: torch.Tensor | None = None, stream=None,
                       ring: torch.Tensor | None = None):
    """Producer + GEMM through the packed-tile ring: x [M, K] bf16 -> out [M, N]
    bf16; returns (out, tensor_scale f32[1], amax f32[1], ring).  The ring
    (slots x nvfp4_ring_slot_bytes(chunk_rows, K) bytes) and the GEMM
    workspace are allocated on the launch stream unless a ring is given."""
    _bits16(x)
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    N = qw.shape[0]
    seg, keep = make_segments(row_start, shift, scale)
    dev = x.device
    st = _torch_stream(stream, dev)
    slot = nvfp4_ring_slot_bytes(chunk_rows, K)
    need = nvfp4_ring_gemm_workspace_bytes(M, chunk_rows, N, K)
    with torch.cuda.stream(st):
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        amax = torch.empty(1, dtype=torch.float32, device=dev)
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if ring is None or ring.numel() * ring.element_size() < slots * slot:
            ring = torch.empty(slots * slot, dtype=torch.uint8, device=dev)
        gws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    nvfp4_modulate_gemm_ring(x, M, K, x.stride(0), seg, workspace(dev, st), ts, amax, ring, slots, chunk_rows, qw,
                             sfw, w_scale, N, out, out.stride(0), gws, need, st)
    del keep
    return out, ts, amax, ring
