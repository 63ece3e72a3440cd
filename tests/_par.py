"""Run the single-threaded oracle over row ranges or element chunks on several
host threads (ctypes releases the GIL).  The maximum over row ranges is exact,
so the results are those of one sequential pass."""
import concurrent.futures as cf
import os

import numpy as np

import oracle

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def _ranges(n, parts):
    parts = max(1, min(parts, n))
    step = (n + parts - 1) // parts
    return [(a, min(n, a + step)) for a in range(0, n, step)]


def _map(fn, items):
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(fn, items))


def amax_merge(values):
    """Maximum of per-range maxima (non-negative bf16 magnitudes, NaN possible)
    as the oracle takes it: over bit patterns, so NaN ranks above Inf above
    every finite value (Python's max() would drop a NaN depending on order)."""
    bits = np.array([np.float32(v) for v in values], np.float32).view(np.uint32)
    return float(bits.max().view(np.float32))


def modulate_quantize(x, seg, m_pad):
    M = x.shape[0]
    x = np.ascontiguousarray(x)
    amax = amax_merge(_map(lambda r: oracle.modulate_amax_rows(x, seg, *r), _ranges(M, 4 * WORKERS)))
    s_g = oracle.tensor_scale(amax)
    parts = _map(lambda r: oracle.modulate_pack_rows(x, seg, s_g, *r), _ranges(m_pad, 4 * WORKERS))
    return (np.float32(s_g), np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            np.float32(amax))


def modulate_pack(x, seg, s_g, r0, r1):
    x = np.ascontiguousarray(x)
    parts = _map(lambda r: oracle.modulate_pack_rows(x, seg, s_g, *r),
                 [(a + r0, b + r0) for a, b in _ranges(r1 - r0, 4 * WORKERS)])
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def swiglu_quantize(gu, m_pad):
    M = gu.shape[0]
    gu = np.ascontiguousarray(gu)
    amax = amax_merge(_map(lambda r: oracle.swiglu_amax_rows(gu, *r), _ranges(M, 4 * WORKERS)))
    s_g = oracle.tensor_scale(amax)
    parts = _map(lambda r: oracle.swiglu_pack_rows(gu, s_g, *r), _ranges(m_pad, 4 * WORKERS))
    return (np.float32(s_g), np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            np.float32(amax))


def swiglu_pack(gu, s_g, r0, r1):
    gu = np.ascontiguousarray(gu)
    parts = _map(lambda r: oracle.swiglu_pack_rows(gu, s_g, *r),
                 [(a + r0, b + r0) for a, b in _ranges(r1 - r0, 4 * WORKERS)])
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def quantize_bf16(y, m_pad=None):
    M = y.shape[0]
    m_pad = M if m_pad is None else m_pad
    y = np.ascontiguousarray(y)
    amax = amax_merge(_map(lambda r: oracle.bf16_amax(y[r[0]:r[1]]), _ranges(M, 4 * WORKERS)))
    s_g = oracle.tensor_scale(amax)
    parts = _map(lambda r: oracle.bf16_pack_rows(y, s_g, *r), _ranges(m_pad, 4 * WORKERS))
    return (np.float32(s_g), np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            np.float32(amax))


def gemm_rows(qa, sfa, a_scale, qw, sfw, w_scale, rows):
    rows = np.asarray(rows, np.int64)
    chunks = [rows[a:b] for a, b in _ranges(rows.size, WORKERS)]
    outs = _map(lambda r: oracle.gemm_rows(qa, sfa, a_scale, qw, sfw, w_scale, r), chunks)
    return np.concatenate(outs, axis=0)


def gemm_bf16_rows(qa, sfa, a_scale, qw, sfw, w_scale, rows):
    rows = np.asarray(rows, np.int64)
    chunks = [rows[a:b] for a, b in _ranges(rows.size, WORKERS)]
    outs = _map(lambda r: oracle.gemm_bf16_rows(qa, sfa, a_scale, qw, sfw, w_scale, r), chunks)
    return np.concatenate(outs, axis=0)


def batch(fn, n, *arrays):
    """fn(*slices) -> array; applied to chunks of the flattened inputs."""
    arrays = [np.ascontiguousarray(a).ravel() for a in arrays]
    outs = _map(lambda r: fn(*[a[r[0]:r[1]] for a in arrays]), _ranges(n, 8 * WORKERS))
    return np.concatenate(outs)
