"""The C ABI library: it loads, exports every entry point its header declares,
and rejects bad arguments synchronously without launching anything (CPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def pkg():
    import nvfp4_activation_quantization_segment_amd as m

    return m


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("nvfp4_modulate_absmax", "nvfp4_modulate_pack", "nvfp4_swiglu_absmax", "nvfp4_swiglu_pack",
              "nvfp4_gemm", "nvfp4_padded_rows", "nvfp4_absmax_workspace_bytes"):
        assert s in syms


def test_library_exports_every_declared_symbol(pkg):
    L = ctypes.CDLL(pkg.LIB_PATH)
    missing = [s for s in declared_symbols() if not hasattr(L, s)]
    assert not missing, missing


def test_library_is_hip_code_for_gfx950(pkg):
    data = open(pkg.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_padded_rows_and_workspace(pkg):
    assert pkg.lib.nvfp4_padded_rows(37810) == 37824
    assert pkg.lib.nvfp4_padded_rows(64) == 64
    assert pkg.lib.nvfp4_padded_rows(1) == 64
    assert pkg.lib.nvfp4_absmax_workspace_bytes() >= 8


FAKE = 1 << 20  # never dereferenced: every call below fails validation first


def _seg(pkg, rows, count=1, ld=64, shift=FAKE, scale=FAKE):
    rs = (ctypes.c_int64 * (count + 1))(*rows)
    return pkg.Segments(count, ctypes.cast(rs, ctypes.POINTER(ctypes.c_int64)), shift, scale, ld), rs


def test_gemm_argument_errors(pkg):
    g = pkg.lib.nvfp4_gemm
    P = FAKE
    assert g(None, P, P, 10, 64, P, P, P, 64, 64, P, 64, None) == 1
    assert g(P, P, P, 0, 64, P, P, P, 64, 64, P, 64, None) == 1
    assert g(P, P, P, 10, 64, P, P, P, 64, 48, P, 64, None) == 2       # K % 64
    assert g(P, P, P, 10, 64, P, P, P, 1 << 20, 1 << 14, P, 1 << 20, None) == 2   # weight past 4 GiB
    assert g(P, P, P, 10, 64, P, P, P, 1 << 18, 1 << 15, P, 1 << 18, None) == 2   # weight of exactly 4 GiB
    assert g(P, P, P, 10, 64, P, P, P, 16, 1 << 26, P, 16, None) == 2  # K > 2^25
    assert g(P, P, P, 10, 64, P, P, P, 40, 64, P, 64, None) == 2       # N % 16
    assert g(P, P, P, 10, 8, P, P, P, 64, 64, P, 64, None) == 1        # M_pad < M
    assert g(P, P, P, 10, 64, P, P, P, 64, 64, P, 32, None) == 1       # ldo < N
    assert g(P + 4, P, P, 10, 64, P, P, P, 64, 64, P, 64, None) == 3   # qa alignment
    assert g(P, P, P, 10, 64, P, P, P, 64, 64, P + 2, 64, None) == 3   # out alignment
    assert g(P, P, P, 10, 64, P, P, P, 64, 64, P, 66, None) == 3       # ldo % 4


def test_gemm_workspace_plan(pkg):
    """The split of the last workgroup wave depends on the shape only: of the
    projection GEMMs only FC2 (3108 tiles of 256x256 = 12 waves of 256 and 36
    tiles) splits, its 36 tail tiles into 7 K ranges of 32 steps."""
    wsb = pkg.lib.nvfp4_gemm_workspace_bytes
    tile = 8 * 128 * 64 * 4  # fp32 partial sums of one 256x256 tile
    assert wsb(37810, 21504, 5376) == 0      # 12432 tiles: tail of 144 > 256/3
    assert wsb(37810, 14336, 5376) == 0      # 8288 tiles: tail of 96 > 256/3
    assert wsb(37810, 5376, 14336) == 36 * 7 * tile
    # an activation past 4 GiB runs in row chunks of 599,040 rows at K = 14336:
    # the full chunk (2340 x 1 tiles: 36 tail tiles in 7 ranges) needs more
    # than the last one (960 rows: 4 tiles in 14 ranges of 16 steps)
    assert wsb(600_000, 256, 14336) == 36 * 7 * tile
    assert wsb(1, 16, 64) == 0               # one K step: nothing to split
    assert wsb(64, 16, 5376) == 11 * tile    # one tile, 84 steps in 11 ranges of 8
    assert wsb(10, 16, 48) == 0              # invalid K


def test_gemm_ws_argument_errors(pkg):
    g = pkg.lib.nvfp4_gemm_ws
    P = FAKE
    need = pkg.lib.nvfp4_gemm_workspace_bytes(64, 16, 5376)
    assert need > 0
    assert g(P, P, P, 64, 64, P, P, P, 16, 5376, P, 16, None, need, None) == 1        # no workspace
    assert g(P, P, P, 64, 64, P, P, P, 16, 5376, P, 16, P, need - 1, None) == 1       # short workspace
    assert g(P, P, P, 64, 64, P, P, P, 16, 5376, P, 16, P + 4, need, None) == 3       # workspace alignment
    assert g(P, P, P, 10, 64, P, P, P, 64, 48, P, 64, P, 1 << 20, None) == 2          # K % 64, as nvfp4_gemm


def test_producer_argument_errors(pkg):
    L = pkg.lib
    seg, keep = _seg(pkg, [0, 10])
    ws = ts = q = s = FAKE
    assert L.nvfp4_modulate_absmax(None, 10, 64, 64, ctypes.byref(seg), ws, ts, None, None) == 1
    assert L.nvfp4_modulate_absmax(FAKE, 10, 40, 40, ctypes.byref(seg), ws, ts, None, None) == 2   # D % 16
    assert L.nvfp4_modulate_absmax(FAKE, 10, 64, 60, ctypes.byref(seg), ws, ts, None, None) == 1   # ldx < D
    assert L.nvfp4_modulate_absmax(FAKE, 10, 64, 68, ctypes.byref(seg), ws, ts, None, None) == 3   # ldx % 8
    assert L.nvfp4_modulate_absmax(FAKE + 8, 10, 64, 64, ctypes.byref(seg), ws, ts, None, None) == 3
    bad, keep2 = _seg(pkg, [0, 9])
    assert L.nvfp4_modulate_absmax(FAKE, 10, 64, 64, ctypes.byref(bad), ws, ts, None, None) == 4
    bad2, keep3 = _seg(pkg, [0, 5, 5, 10], count=3)
    assert L.nvfp4_modulate_absmax(FAKE, 10, 64, 64, ctypes.byref(bad2), ws, ts, None, None) == 4
    many, keep4 = _seg(pkg, list(range(18)), count=17)
    assert L.nvfp4_modulate_absmax(FAKE, 17, 64, 64, ctypes.byref(many), ws, ts, None, None) == 4
    assert L.nvfp4_modulate_pack(FAKE, 10, 64, 64, ctypes.byref(seg), ts, q, s, 32, None) == 2     # M_pad
    assert L.nvfp4_modulate_pack(FAKE, 10, 64, 64, ctypes.byref(seg), ts, q + 1, s, 64, None) == 3
    mq = L.nvfp4_modulate_quantize
    assert mq(None, 10, 64, 64, ctypes.byref(seg), ws, ts, None, q, s, 64, None) == 1
    assert mq(FAKE, 10, 40, 40, ctypes.byref(seg), ws, ts, None, q, s, 64, None) == 2            # D % 16
    assert mq(FAKE, 10, 64, 64, ctypes.byref(bad), ws, ts, None, q, s, 64, None) == 4            # segments
    assert mq(FAKE, 10, 64, 64, ctypes.byref(seg), None, ts, None, q, s, 64, None) == 1          # workspace
    assert mq(FAKE, 10, 64, 64, ctypes.byref(seg), ws, ts, None, q, s, 32, None) == 2            # M_pad
    assert mq(FAKE, 10, 64, 64, ctypes.byref(seg), ws, ts, None, q + 1, s, 64, None) == 3        # qdata
    assert mq(FAKE, 10, 64, 64, ctypes.byref(seg), ws, ts, FAKE + 2, q, s, 64, None) == 3        # amax_out
    assert L.nvfp4_quantize(None, 10, 64, 64, ws, ts, None, q, s, 64, None) == 1
    assert L.nvfp4_quantize(FAKE, 10, 40, 40, ws, ts, None, q, s, 64, None) == 2           # D % 16
    assert L.nvfp4_quantize(FAKE, 10, 64, 64, None, ts, None, q, s, 64, None) == 1         # workspace
    assert L.nvfp4_quantize(FAKE, 10, 64, 64, ws, ts, None, q, s, 32, None) == 2           # M_pad
    assert L.nvfp4_quantize(FAKE, 10, 64, 64, ws, ts, None, q + 2, s, 64, None) == 3       # qdata
    assert L.nvfp4_swiglu_absmax(FAKE, FAKE, 10, 24, 48, ws, ts, None, None) == 2
    assert L.nvfp4_swiglu_pack(FAKE, None, 10, 32, 64, ts, q, s, 64, None) == 1
    sq = L.nvfp4_swiglu_quantize
    assert sq(FAKE, None, 10, 32, 64, ws, ts, None, q, s, 64, None) == 1                  # up
    assert sq(FAKE, FAKE, 10, 24, 48, ws, ts, None, q, s, 64, None) == 2                  # F % 16
    assert sq(FAKE, FAKE, 10, 32, 64, None, ts, None, q, s, 64, None) == 1                # workspace
    assert sq(FAKE, FAKE, 10, 32, 64, ws, ts, None, q, s, 32, None) == 2                  # M_pad
    assert sq(FAKE, FAKE, 10, 32, 64, ws, ts, None, q + 1, s, 64, None) == 3              # qdata


def test_gate_residual_argument_errors(pkg):
    g = pkg.lib.nvfp4_gemm_gate_residual
    P = FAKE
    rs = (ctypes.c_int64 * 3)(0, 5, 10)
    gates = pkg.RowGates(2, ctypes.cast(rs, ctypes.POINTER(ctypes.c_int64)), P, 64)
    args = lambda **k: dict(dict(M=10, N=64, K=64, gates=ctypes.byref(gates), res=P, ldr=64, out=P, ldo=64), **k)  # noqa: E731
    call = lambda a: g(P, P, P, a["M"], 64, P, P, P, a["N"], a["K"], a["gates"], a["res"], a["ldr"], a["out"],  # noqa: E731
                       a["ldo"], P, 1 << 20, None)
    assert call(args(res=None)) == 1                   # no residual
    assert call(args(gates=None)) == 1                 # no gate table
    assert call(args(K=48)) == 2                       # K % 64, as nvfp4_gemm
    assert call(args(ldr=60)) == 1                     # ldr < N
    assert call(args(ldr=66)) == 3                     # ldr % 4
    assert call(args(res=P + 4)) == 3                  # residual alignment
    bad = (ctypes.c_int64 * 3)(0, 5, 9)
    gb = pkg.RowGates(2, ctypes.cast(bad, ctypes.POINTER(ctypes.c_int64)), P, 64)
    assert call(args(gates=ctypes.byref(gb))) == 4     # last row != M
    zero = pkg.RowGates(0, ctypes.cast(rs, ctypes.POINTER(ctypes.c_int64)), P, 64)
    assert call(args(gates=ctypes.byref(zero))) == 4   # no segments
    short = pkg.RowGates(2, ctypes.cast(rs, ctypes.POINTER(ctypes.c_int64)), P, 32)
    assert call(args(gates=ctypes.byref(short))) == 1  # gate ld < N


def test_status_strings(pkg):
    for st in range(6):
        assert pkg.lib.nvfp4_status_string(st)


def test_barrier_settings_round_trip(pkg):
    """The single launches' barrier settings: each setter returns the value it
    replaces (defaults 1 s and 100 us); host state only, nothing launched."""
    assert pkg.lib.nvfp4_absmax_workspace_bytes() == 256 + 2 * 8 * 1024
    t0 = pkg.set_barrier_timeout_us(250)
    h0 = pkg.set_barrier_help_us(7)
    try:
        assert pkg.set_barrier_timeout_us(0) == 250
        assert pkg.set_barrier_help_us(0) == 7
        assert pkg.set_barrier_timeout_us(2**40) == 0
        assert pkg.set_barrier_timeout_us(1000000) == 2**40
    finally:
        pkg.set_barrier_timeout_us(t0)
        pkg.set_barrier_help_us(h0)
    assert (t0, h0) == (1000000, 100)
