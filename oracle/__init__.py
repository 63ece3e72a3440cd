"""NVFP4 activation-quantization oracle -- TEST INFRASTRUCTURE ONLY.

A plain, single-threaded C implementation (``nvfp4_oracle.c``) of what the
producer and the block-scaled GEMM compute, loaded with ctypes.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product path never does.  It shares no code with the HIP
library.

Functions take and return numpy arrays: bf16 tensors are ``uint16`` bit
patterns, QDATA/SFA are ``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    cmd = ["gcc", *CFLAGS, _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_U8 = ctypes.c_uint8
_U16 = ctypes.c_uint16

_SIGS = {
    "ora_bf16_to_f32": (_F, [_U16]),
    "ora_f32_to_bf16": (_U16, [_F]),
    "ora_e4m3_value": (ctypes.c_double, [_U8]),
    "ora_e4m3_encode": (_U8, [_F]),
    "ora_e2m1_value": (ctypes.c_double, [_U8]),
    "ora_e2m1_encode": (_U8, [_F]),
    "ora_modulate": (_U16, [_U16, _U16, _U16]),
    "ora_exp_neg": (_F, [_U16]),
    "ora_silu_bf16": (_U16, [_U16]),
    "ora_swiglu": (_U16, [_U16, _U16]),
    "ora_tensor_scale": (_F, [_F]),
    "ora_block_scale": (_U8, [_F, _F]),
    "ora_element_code": (_U8, [_U16, _U8, _F]),
    "ora_modulate_amax": (_F, [_P, _I64, _I64, _I64, _I32, _P, _P, _P, _I64]),
    "ora_modulate_pack_rows": (None, [_P, _I64, _I64, _I64, _I32, _P, _P, _P, _I64, _F, _I64, _I64, _P, _P]),
    "ora_swiglu_amax": (_F, [_P, _P, _I64, _I64, _I64]),
    "ora_swiglu_pack_rows": (None, [_P, _P, _I64, _I64, _I64, _F, _I64, _I64, _P, _P]),
    "ora_bf16_amax": (_F, [_P, _I64, _I64, _I64]),
    "ora_bf16_pack_rows": (None, [_P, _I64, _I64, _I64, _F, _I64, _I64, _P, _P]),
    "ora_gemm_rows": (None, [_P, _P, _F, _P, _P, _F, _I64, _I64, _P, _I64, _P]),
    "ora_gemm_bf16_rows": (None, [_P, _P, _F, _P, _P, _F, _I64, _I64, _P, _I64, _P]),
    "ora_gate_residual": (_U16, [_U16, _U16, _U16]),
    "ora_gate_residual_rows": (None, [_P, _I64, _I64, _I64, _I32, _P, _P, _I64, _P, _I64, _P, _I64]),
    "ora_modulate_amax_rows": (_F, [_P, _I64, _I64, _I32, _P, _P, _P, _I64, _I64, _I64]),
    "ora_swiglu_amax_rows": (_F, [_P, _P, _I64, _I64, _I64, _I64]),
    "ora_modulate_batch": (None, [_P, _P, _P, _I64, _P]),
    "ora_swiglu_batch": (None, [_P, _P, _I64, _P]),
    "ora_block_scale_batch": (None, [_P, _I64, _F, _P]),
    "ora_element_code_batch": (None, [_P, _P, _I64, _F, _P]),
    "ora_e2m1_encode_batch": (None, [_P, _I64, _P]),
    "ora_e4m3_encode_batch": (None, [_P, _I64, _P]),
}


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def padded_rows(m: int) -> int:
    """Rows zero-padded to a multiple of 64 (37,810 -> 37,824)."""
    return (m + 63) // 64 * 64


# --------------------------------------------------------------------------
# scalar helpers (thin wrappers)
# --------------------------------------------------------------------------
def f32_to_bf16(f: float) -> int:
    return int(lib().ora_f32_to_bf16(float(np.float32(f))))


def bf16_to_f32(h: int) -> float:
    return float(lib().ora_bf16_to_f32(int(h)))


def e4m3_encode(t: float) -> int:
    return int(lib().ora_e4m3_encode(float(np.float32(t))))


def e4m3_value(code: int) -> float:
    return float(lib().ora_e4m3_value(int(code)))


def e2m1_encode(v: float) -> int:
    return int(lib().ora_e2m1_encode(float(np.float32(v))))


def e2m1_value(code: int) -> float:
    return float(lib().ora_e2m1_value(int(code)))


def modulate(x: int, scale: int, shift: int) -> int:
    return int(lib().ora_modulate(int(x), int(scale), int(shift)))


def silu_bf16(g: int) -> int:
    return int(lib().ora_silu_bf16(int(g)))


def swiglu(g: int, u: int) -> int:
    return int(lib().ora_swiglu(int(g), int(u)))


def exp_neg(g: int) -> float:
    return float(lib().ora_exp_neg(int(g)))


def tensor_scale(amax: float) -> float:
    return float(lib().ora_tensor_scale(float(np.float32(amax))))


def block_scale(a16: float, s_g: float) -> int:
    return int(lib().ora_block_scale(float(np.float32(a16)), float(np.float32(s_g))))


def element_code(y: int, sf: int, s_g: float) -> int:
    return int(lib().ora_element_code(int(y), int(sf), float(np.float32(s_g))))


# --------------------------------------------------------------------------
# tensor passes
# --------------------------------------------------------------------------
class Segments:
    """Contiguous row ranges with per-segment bf16 shift/scale rows [S, D]."""

    def __init__(self, row_start, shift: np.ndarray, scale: np.ndarray):
        self.row_start = np.ascontiguousarray(np.asarray(row_start, dtype=np.int64))
        self.shift = _c(shift, np.uint16)
        self.scale = _c(scale, np.uint16)
        assert self.shift.shape == self.scale.shape and self.shift.ndim == 2
        assert self.row_start.shape[0] == self.shift.shape[0] + 1

    @property
    def count(self) -> int:
        return int(self.shift.shape[0])


def modulate_amax(x: np.ndarray, seg: Segments) -> float:
    x = _c(x, np.uint16)
    M, D = x.shape
    return float(lib().ora_modulate_amax(_ptr(x), M, D, D, seg.count, _ptr(seg.row_start),
                                         _ptr(seg.shift), _ptr(seg.scale), seg.shift.shape[1]))


def modulate_amax_rows(x: np.ndarray, seg: Segments, r0: int, r1: int) -> float:
    """max |y| over rows [r0, r1) of x (row indices of the full tensor)."""
    x = _c(x, np.uint16)
    M, D = x.shape
    return float(lib().ora_modulate_amax_rows(_ptr(x), D, D, seg.count, _ptr(seg.row_start), _ptr(seg.shift),
                                              _ptr(seg.scale), seg.shift.shape[1], r0, r1))


def swiglu_amax_rows(gu: np.ndarray, r0: int, r1: int) -> float:
    gu = _c(gu, np.uint16)
    M, F2 = gu.shape
    F = F2 // 2
    base = gu.ctypes.data
    return float(lib().ora_swiglu_amax_rows(ctypes.c_void_p(base), ctypes.c_void_p(base + 2 * F), F, F2, r0, r1))


def modulate_pack_rows(x: np.ndarray, seg: Segments, s_g: float, r0: int, r1: int):
    x = _c(x, np.uint16)
    M, D = x.shape
    q = np.empty((r1 - r0, D // 2), np.uint8)
    s = np.empty((r1 - r0, D // 16), np.uint8)
    lib().ora_modulate_pack_rows(_ptr(x), M, D, D, seg.count, _ptr(seg.row_start), _ptr(seg.shift),
                                 _ptr(seg.scale), seg.shift.shape[1], float(np.float32(s_g)), r0, r1,
                                 _ptr(q), _ptr(s))
    return q, s


def modulate_quantize(x: np.ndarray, seg: Segments, m_pad: int | None = None):
    """Full two-phase producer: returns (s_g, qdata [M_pad, D/2], sfa [M_pad, D/16], amax)."""
    M = x.shape[0]
    m_pad = padded_rows(M) if m_pad is None else m_pad
    amax = modulate_amax(x, seg)
    s_g = tensor_scale(amax)
    q, s = modulate_pack_rows(x, seg, s_g, 0, m_pad)
    return np.float32(s_g), q, s, np.float32(amax)


def swiglu_amax(gu: np.ndarray) -> float:
    """gu: [M, 2F] bf16 with gate = first F columns, up = last F columns."""
    gu = _c(gu, np.uint16)
    M, F2 = gu.shape
    F = F2 // 2
    base = gu.ctypes.data
    return float(lib().ora_swiglu_amax(ctypes.c_void_p(base), ctypes.c_void_p(base + 2 * F), M, F, F2))


def swiglu_pack_rows(gu: np.ndarray, s_g: float, r0: int, r1: int):
    gu = _c(gu, np.uint16)
    M, F2 = gu.shape
    F = F2 // 2
    q = np.empty((r1 - r0, F // 2), np.uint8)
    s = np.empty((r1 - r0, F // 16), np.uint8)
    base = gu.ctypes.data
    lib().ora_swiglu_pack_rows(ctypes.c_void_p(base), ctypes.c_void_p(base + 2 * F), M, F, F2,
                               float(np.float32(s_g)), r0, r1, _ptr(q), _ptr(s))
    return q, s


def swiglu_quantize(gu: np.ndarray, m_pad: int | None = None):
    M = gu.shape[0]
    m_pad = padded_rows(M) if m_pad is None else m_pad
    amax = swiglu_amax(gu)
    s_g = tensor_scale(amax)
    q, s = swiglu_pack_rows(gu, s_g, 0, m_pad)
    return np.float32(s_g), q, s, np.float32(amax)


def bf16_amax(y: np.ndarray) -> float:
    y = _c(y, np.uint16)
    M, D = y.shape
    return float(lib().ora_bf16_amax(_ptr(y), M, D, D))


def bf16_pack_rows(y: np.ndarray, s_g: float, r0: int, r1: int):
    y = _c(y, np.uint16)
    M, D = y.shape
    q = np.empty((r1 - r0, D // 2), np.uint8)
    s = np.empty((r1 - r0, D // 16), np.uint8)
    lib().ora_bf16_pack_rows(_ptr(y), M, D, D, float(np.float32(s_g)), r0, r1, _ptr(q), _ptr(s))
    return q, s


def quantize_bf16(y: np.ndarray, m_pad: int | None = None):
    """Plain NVFP4 quantizer of an already-formed bf16 tensor (used to prepack weights)."""
    M = y.shape[0]
    m_pad = M if m_pad is None else m_pad
    amax = bf16_amax(y)
    s_g = tensor_scale(amax)
    q, s = bf16_pack_rows(y, s_g, 0, m_pad)
    return np.float32(s_g), q, s, np.float32(amax)


def gemm_rows(qa, sfa, a_scale, qw, sfw, w_scale, rows) -> np.ndarray:
    """FP64 reference outputs [len(rows), N] (alpha applied, not rounded to bf16)."""
    qa = _c(qa, np.uint8)
    sfa = _c(sfa, np.uint8)
    qw = _c(qw, np.uint8)
    sfw = _c(sfw, np.uint8)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    N, Kh = qw.shape
    K = Kh * 2
    assert qa.shape[1] == Kh and sfa.shape[1] == K // 16 and sfw.shape == (N, K // 16)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < qa.shape[0])
    out = np.empty((rows.size, N), np.float64)
    lib().ora_gemm_rows(_ptr(qa), _ptr(sfa), float(np.float32(a_scale)), _ptr(qw), _ptr(sfw),
                        float(np.float32(w_scale)), N, K, _ptr(rows), rows.size, _ptr(out))
    return out


def gemm_bf16_rows(qa, sfa, a_scale, qw, sfw, w_scale, rows) -> np.ndarray:
    """BF16 outputs [len(rows), N] (uint16) with the sum rounded once to binary32:
    the GEMM's bf16 output whenever its binary32 accumulation is exact."""
    qa = _c(qa, np.uint8)
    sfa = _c(sfa, np.uint8)
    qw = _c(qw, np.uint8)
    sfw = _c(sfw, np.uint8)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    N, Kh = qw.shape
    K = Kh * 2
    assert qa.shape[1] == Kh and sfa.shape[1] == K // 16 and sfw.shape == (N, K // 16)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < qa.shape[0])
    out = np.empty((rows.size, N), np.uint16)
    lib().ora_gemm_bf16_rows(_ptr(qa), _ptr(sfa), float(np.float32(a_scale)), _ptr(qw), _ptr(sfw),
                             float(np.float32(w_scale)), N, K, _ptr(rows), rows.size, _ptr(out))
    return out


def gate_residual(o: int, gate: int, residual: int) -> int:
    """bf16(residual + bf16(gate * o)) for one element."""
    return int(lib().ora_gate_residual(int(o), int(gate), int(residual)))


def gate_residual_rows(o, row_start, gate, residual) -> np.ndarray:
    """The exact residual epilogue over o [M, N] (uint16 bf16 patterns): row m
    uses gate row s of its segment [row_start[s], row_start[s+1])."""
    o = _c(o, np.uint16)
    gate = _c(gate, np.uint16)
    residual = _c(residual, np.uint16)
    rs = np.ascontiguousarray(np.asarray(row_start, dtype=np.int64))
    M, N = o.shape
    assert gate.shape[1] == N and residual.shape == (M, N) and rs[0] == 0 and rs[-1] == M
    out = np.empty((M, N), np.uint16)
    lib().ora_gate_residual_rows(_ptr(o), M, N, N, rs.size - 1, _ptr(rs), _ptr(gate), N, _ptr(residual), N,
                                 _ptr(out), N)
    return out


def gemm_tolerance_ok(gpu: np.ndarray, ref: np.ndarray):
    """|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), rms over the checked set.

    Returns (ok, worst_ratio) where worst_ratio = max |gpu-ref| / bound."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = 2.0 ** -7 * np.abs(ref) + 1e-3 * rms
    err = np.abs(gpu - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(np.all(err <= bound)), worst


# --------------------------------------------------------------------------
# elementwise batches
# --------------------------------------------------------------------------
def modulate_batch(x, scale, shift) -> np.ndarray:
    x, scale, shift = (_c(a, np.uint16).ravel() for a in (x, scale, shift))
    y = np.empty(x.size, np.uint16)
    lib().ora_modulate_batch(_ptr(x), _ptr(scale), _ptr(shift), x.size, _ptr(y))
    return y


def swiglu_batch(g, u) -> np.ndarray:
    g, u = (_c(a, np.uint16).ravel() for a in (g, u))
    h = np.empty(g.size, np.uint16)
    lib().ora_swiglu_batch(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def block_scale_batch(a16_bits, s_g: float) -> np.ndarray:
    a = _c(a16_bits, np.uint16).ravel()
    out = np.empty(a.size, np.uint8)
    lib().ora_block_scale_batch(_ptr(a), a.size, float(np.float32(s_g)), _ptr(out))
    return out


def element_code_batch(y, sf, s_g: float) -> np.ndarray:
    y = _c(y, np.uint16).ravel()
    sf = _c(sf, np.uint8).ravel()
    out = np.empty(y.size, np.uint8)
    lib().ora_element_code_batch(_ptr(y), _ptr(sf), y.size, float(np.float32(s_g)), _ptr(out))
    return out


def e2m1_batch(v) -> np.ndarray:
    v = _c(v, np.float32).ravel()
    out = np.empty(v.size, np.uint8)
    lib().ora_e2m1_encode_batch(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_batch(t) -> np.ndarray:
    t = _c(t, np.float32).ravel()
    out = np.empty(t.size, np.uint8)
    lib().ora_e4m3_encode_batch(_ptr(t), t.size, _ptr(out))
    return out
