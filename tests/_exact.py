"""Exact rational arithmetic rounded once to binary32, vectorised with numpy
integers (test infrastructure for the oracle's pins).

A positive finite binary32 value is an integer mantissa m and exponent e with
value m * 2^e.  The quotient and product below are formed exactly as integer
ratios and rounded to the nearest binary32 value, ties to the even significand,
with gradual underflow and overflow to infinity, following IEEE 754's
definition of a correctly rounded result.  No floating-point division or
multiplication is involved, so these pins do not retrace the oracle's own
binary32 operations.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def decompose(x) -> tuple[np.ndarray, np.ndarray]:
    """binary32 values (finite, >= 0) -> (m, e) with x = m * 2^e, m < 2^24 odd
    (or 0)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.int64)
    E = (b >> 23) & 0xFF
    F = b & 0x7FFFFF
    assert np.all(E < 0xFF), "finite inputs only"
    assert np.all((b >> 31) == 0), "non-negative inputs only"
    m = np.where(E == 0, F, F | (1 << 23))
    e = np.where(E == 0, -149, E - 150)
    # drop trailing zero bits, so that products of short significands stay small
    tz = np.where(m == 0, 0, _bitlen(m & -m) - 1)
    return m >> tz, e + tz


def _bitlen(v: np.ndarray) -> np.ndarray:
    """Bit length of non-negative integers below 2^53."""
    v = np.asarray(v, np.int64)
    _, ex = np.frexp(v.astype(np.float64))
    return np.where(v == 0, 0, ex).astype(np.int64)


def round_ratio(n, d, e) -> np.ndarray:
    """The binary32 nearest to (n / d) * 2^e, ties to even, for integers
    0 <= n < 2^31 (or < 2^50 when d == 1), 1 <= d < 2^31 and integer e."""
    n = np.asarray(n, np.int64)
    d = np.asarray(d, np.int64)
    e = np.asarray(e, np.int64)
    n, d, e = np.broadcast_arrays(n, d, e)
    assert np.all(d >= 1) and np.all(n >= 0)
    bn = _bitlen(n)
    bd = _bitlen(d)
    k = np.maximum(0, 27 + bd - bn)            # quotient gets 26 or more bits
    assert np.all(bn + k < 63)
    num = n << k
    Q = num // d
    R = num - Q * d
    eq = e - k                                   # value = (Q + R/d) * 2^eq
    bq = _bitlen(Q)
    lead = eq + bq - 1
    ulp = np.maximum(lead - 23, -149)            # binary32 grid at that magnitude
    shift = np.minimum(ulp - eq, 62)
    assert np.all((shift >= 2) | (n == 0))
    shift = np.maximum(shift, 2)
    kept = Q >> shift
    rem = Q - (kept << shift)
    half = np.int64(1) << (shift - 1)
    up = (rem > half) | ((rem == half) & ((R != 0) | ((kept & 1) == 1)))
    kept = kept + up
    with np.errstate(over="ignore"):
        out = np.ldexp(kept.astype(np.float64), ulp.astype(np.int64)).astype(np.float32)
    return np.where(n == 0, np.float32(0.0), out)


def div32(a, b) -> np.ndarray:
    """RN32(a / b) for positive finite binary32 a and b (a may be 0)."""
    am, ae = decompose(a)
    bm, be = decompose(b)
    assert np.all(bm > 0)
    return round_ratio(am, bm, ae - be)


def mul32(a, b) -> np.ndarray:
    """RN32(a * b) for non-negative finite binary32 a and b."""
    am, ae = decompose(a)
    bm, be = decompose(b)
    return round_ratio(am * bm, 1, ae + be)


def div32_int(a, c: int) -> np.ndarray:
    """RN32(a / c) for a positive integer constant c (exact, one rounding)."""
    am, ae = decompose(a)
    return round_ratio(am, c, ae)


def rn32_fraction(q: Fraction) -> np.float32:
    """Slow scalar reference: nearest binary32 to a non-negative Fraction, ties
    to even, by comparison with the two neighbours (used to check round_ratio)."""
    if q == 0:
        return np.float32(0.0)
    with np.errstate(over="ignore"):
        lo = np.float32(float(q))               # within one ulp of q
    cands = [np.nextafter(lo, np.float32(0)), lo, np.nextafter(lo, np.float32(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            # the value just above the largest finite one, for overflow
            cv = Fraction(2) ** 128
        else:
            cv = Fraction(float(c))
        dist = abs(cv - q)
        key = (dist, int(np.float32(c).view(np.uint32)) & 1 if np.isfinite(c) else 0)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])
