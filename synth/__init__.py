"""Seeded synthetic workloads for the NVFP4 producer and GEMM.

This module only draws random numbers (``synth.c``, a counter-based
generator) and knows the shapes of the workloads; it holds none of the
quantizer's arithmetic.  It is the one module that both the oracle-side tests
and the HIP-side tests and benchmark draw inputs from.

Workloads (shapes of the pages' H3 block at 37,810 tokens;
synthetic data stands in for the captured activations, which are absent):

=========  =====================================================================
tiny       x [256,512] ~N(0,1), 1% -> +-U[50,300], x[100,256:272] = 0; segments
           rows [0,192) and [192,256); shift/scale [2,512] ~N(0,0.1);
           weight [1024,512] ~N(0,0.02)
producer   x [37810,5376] ~N(0,1), 0.1% -> 20 * t3; segments [0,31000),
           [31000,37810); shift/scale [2,5376] ~N(0,0.1)
qkv        producer inputs; weight [21504,5376] ~N(0,0.02)
fc1        x of producer; own shift/scale; weight [14336,5376] ~N(0,0.02)
fc2        gate/up [37810, 2*14336] ~N(0,1); weight [5376,14336] ~N(0,0.01)
=========  =====================================================================

Streams: t=0 activation, 1 shift, 2 scale, 3 weight, 4 outlier mask,
5 outlier value, 6 row sampler.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

T_X, T_SHIFT, T_SCALE, T_WEIGHT, T_OUT_MASK, T_OUT_VAL, T_ROWS, T_GATE, T_RESIDUAL = range(9)


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", _SRC, "-o", _LIB_PATH + ".tmp",
           "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, d, p, i = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        L.synth_normal_bf16.argtypes = [u64, u64, i64, i64, d, p, i]
        L.synth_outliers_uniform_bf16.argtypes = [u64, u64, u64, i64, i64, d, d, d, p, i]
        L.synth_outliers_t3_bf16.argtypes = [u64, u64, u64, i64, i64, d, d, p, i]
        L.synth_uniform_f64.argtypes = [u64, u64, i64, i64, p, i]
        for f in (L.synth_normal_bf16, L.synth_outliers_uniform_bf16, L.synth_outliers_t3_bf16,
                  L.synth_uniform_f64):
            f.restype = None
        _lib = L
    return _lib


_THREADS: int | None = None


def set_threads(n: int | None) -> None:
    """Generate with n threads (None: the default).  The values do not depend
    on it: every element is a function of its index alone."""
    global _THREADS
    _THREADS = n


def _threads() -> int:
    if _THREADS is not None:
        return max(1, min(64, _THREADS))
    # The GPU host gives one GPU's share of its cores (16); never more.
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(c: int, t: int, shape, sigma: float, out: np.ndarray | None = None) -> np.ndarray:
    n = int(np.prod(shape))
    a = np.empty(shape, np.uint16) if out is None else out
    assert a.dtype == np.uint16 and a.flags.c_contiguous and a.size == n
    _L().synth_normal_bf16(c, t, 0, n, sigma, a.ctypes.data_as(ctypes.c_void_p), _threads())
    return a


def add_outliers_uniform(a: np.ndarray, c: int, p: float, lo: float, hi: float) -> np.ndarray:
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    _L().synth_outliers_uniform_bf16(c, T_OUT_MASK, T_OUT_VAL, 0, a.size, p, lo, hi,
                                     a.ctypes.data_as(ctypes.c_void_p), _threads())
    return a


def add_outliers_t3(a: np.ndarray, c: int, p: float, mult: float) -> np.ndarray:
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    _L().synth_outliers_t3_bf16(c, T_OUT_MASK, T_OUT_VAL, 0, a.size, p, mult,
                                a.ctypes.data_as(ctypes.c_void_p), _threads())
    return a


def uniform(c: int, t: int, n: int) -> np.ndarray:
    a = np.empty(n, np.float64)
    _L().synth_uniform_f64(c, t, 0, n, a.ctypes.data_as(ctypes.c_void_p), _threads())
    return a


def sample_rows(c: int, M: int, k: int, must=()) -> np.ndarray:
    """Sorted distinct rows: the listed boundary rows plus seeded ones, k total."""
    rows = {int(r) for r in must if 0 <= int(r) < M}
    u = uniform(c, T_ROWS, 4 * k + 64)
    j = 0
    while len(rows) < min(k, M) and j < u.size:
        rows.add(int(u[j] * M))
        j += 1
    return np.array(sorted(rows), np.int64)


@dataclass
class Workload:
    """One synthetic configuration.  ``kind`` is 'modulate', 'swiglu' or
    'plain' (quantized without modulation)."""
    name: str
    kind: str
    M: int
    K: int                      # activation width fed to the GEMM (D, or F for swiglu)
    N: int | None               # GEMM output width (None: producer only)
    c_x: int                    # config seed of the activation
    c_seg: int = 0              # config seed of shift/scale
    c_w: int = 0                # config seed of the weight
    x_sigma: float = 1.0
    seg_sigma: float = 0.1
    w_sigma: float = 0.02
    row_start: tuple = ()
    outliers: tuple = ()        # ('uniform', p, lo, hi) or ('t3', p, mult)
    zero_block: tuple = ()      # (row, col0, col1) zeroed in x
    boundary_rows: tuple = field(default_factory=tuple)

    @property
    def m_pad(self) -> int:
        return (self.M + 63) // 64 * 64

    def x(self) -> np.ndarray:
        """Producer input [M, K] bf16 bits (modulation or plain quantizer)."""
        assert self.kind in ("modulate", "plain")
        a = normal_bf16(self.c_x, T_X, (self.M, self.K), self.x_sigma)
        self._outliers(a, self.c_x)
        if self.zero_block:
            r, c0, c1 = self.zero_block
            a[r, c0:c1] = 0
        return a

    def gate_up(self) -> np.ndarray:
        """SwiGLU input [M, 2K] bf16 bits: gate = first K columns, up = last K."""
        assert self.kind == "swiglu"
        a = normal_bf16(self.c_x, T_X, (self.M, 2 * self.K), self.x_sigma)
        self._outliers(a, self.c_x)
        return a

    def _outliers(self, a, c):
        if not self.outliers:
            return
        if self.outliers[0] == "uniform":
            add_outliers_uniform(a, c, *self.outliers[1:])
        elif self.outliers[0] == "t3":
            add_outliers_t3(a, c, *self.outliers[1:])
        else:  # pragma: no cover
            raise ValueError(self.outliers)

    def segments(self):
        """(row_start int64 [S+1], shift [S,K], scale [S,K]) bf16 bits."""
        S = len(self.row_start) - 1
        shift = normal_bf16(self.c_seg, T_SHIFT, (S, self.K), self.seg_sigma)
        scale = normal_bf16(self.c_seg, T_SCALE, (S, self.K), self.seg_sigma)
        return np.array(self.row_start, np.int64), shift, scale

    def weight(self) -> np.ndarray:
        """GEMM weight [N, K] bf16 bits (quantized to NVFP4 before use)."""
        assert self.N is not None
        return normal_bf16(self.c_w, T_WEIGHT, (self.N, self.K), self.w_sigma)

    def gates(self):
        """(row_start int64 [S+1], gate [S, N]) bf16 bits for the residual
        epilogue: gates ~ N(1, seg_sigma) per segment and output column."""
        S = len(self.row_start) - 1
        g = normal_bf16(self.c_seg, T_GATE, (S, self.N), self.seg_sigma)
        # gate = 1 + N(0, sigma): shift the binary32 values by 1, then round to
        # bf16 (nearest, ties to even; every value here is finite)
        u = ((g.astype(np.uint32) << 16).view(np.float32) + np.float32(1.0)).view(np.uint32)
        return np.array(self.row_start, np.int64), ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

    def residual(self) -> np.ndarray:
        """Residual stream [M, N] bf16 bits, N(0, 1)."""
        return normal_bf16(self.c_seg, T_RESIDUAL, (self.M, self.N), 1.0)

    def inputs(self) -> dict:
        """Every generated input of the workload, by name (bf16 bits, except
        the int64 segment bounds)."""
        out = {}
        if self.kind == "swiglu":
            out["gate_up"] = self.gate_up()
        else:
            out["x"] = self.x()
        if self.kind == "modulate":
            out["row_start"], out["shift"], out["scale"] = self.segments()
        if self.N is not None:
            out["weight"] = self.weight()
        if self.kind == "plain" and self.N is not None:
            out["row_start"], out["gate"] = self.gates()
            out["residual"] = self.residual()
        return out

    def check_rows(self, k: int = 64) -> np.ndarray:
        """GEMM rows checked at full size: boundary rows plus seeded rows."""
        return sample_rows(self.c_x, self.M, k, self.boundary_rows)


M_CANON = 37810
_BOUNDARY = (0, 1, 63, 64, 30999, 31000, 37807, 37808, 37809)

WORKLOADS = {
    "tiny": Workload("tiny", "modulate", 256, 512, 1024, c_x=1, c_seg=1, c_w=1, w_sigma=0.02,
                     row_start=(0, 192, 256), outliers=("uniform", 0.01, 50.0, 300.0),
                     zero_block=(100, 256, 272), boundary_rows=(0, 1, 63, 64, 191, 192, 255)),
    "producer": Workload("producer", "modulate", M_CANON, 5376, None, c_x=2, c_seg=2,
                         row_start=(0, 31000, M_CANON), outliers=("t3", 0.001, 20.0),
                         boundary_rows=_BOUNDARY),
    "qkv": Workload("qkv", "modulate", M_CANON, 5376, 21504, c_x=2, c_seg=2, c_w=3, w_sigma=0.02,
                    row_start=(0, 31000, M_CANON), outliers=("t3", 0.001, 20.0),
                    boundary_rows=_BOUNDARY),
    "fc1": Workload("fc1", "modulate", M_CANON, 5376, 14336, c_x=2, c_seg=4, c_w=4, w_sigma=0.02,
                    row_start=(0, 31000, M_CANON), outliers=("t3", 0.001, 20.0),
                    boundary_rows=_BOUNDARY),
    "fc2": Workload("fc2", "swiglu", M_CANON, 14336, 5376, c_x=5, c_w=5, w_sigma=0.01,
                    boundary_rows=_BOUNDARY),
    # attention output: attention values [M, 7168] through the plain quantizer,
    # projected to the model width 5376 with the residual epilogue
    "attn_out": Workload("attn_out", "plain", M_CANON, 7168, 5376, c_x=6, c_seg=6, c_w=6, w_sigma=0.02,
                         row_start=(0, 31000, M_CANON), outliers=("t3", 0.001, 20.0),
                         boundary_rows=_BOUNDARY),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def identity_segments(rows: int, K: int):
    """One segment covering ``rows`` rows whose modulation is the identity:
    scale = +0 (so scale + 1 = 1) and shift = -0 (x + -0 = x for every x,
    including -0).  Returns (row_start, shift, scale) as bf16 bits."""
    return (np.array([0, rows], np.int64),
            np.full((1, K), 0x8000, np.uint16),  # shift = -0
            np.zeros((1, K), np.uint16))         # scale = +0
