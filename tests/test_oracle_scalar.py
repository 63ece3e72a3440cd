"""Pins for the oracle's scalar steps (CPU only).

Each test checks the oracle against something other than itself: a published
format table, a library routine (torch's float8/bf16 conversions and bf16
arithmetic), multiprecision arithmetic, a closed form, or brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def bf16_to_f32_np(h):
    return (np.asarray(h, np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# vectorised wrappers (ctypes per element; sizes kept modest)
# --------------------------------------------------------------------------
def _vec(fn, *arrays, dtype):
    out = np.empty(len(arrays[0]), dtype)
    for i, args in enumerate(zip(*arrays)):
        out[i] = fn(*args)
    return out


# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------
def test_e2m1_decode_table(ora):
    vals = _gold("e2m1_values.json")["values"]
    for c in range(16):
        want = vals[c & 7] * (-1.0 if c & 8 else 1.0)
        assert ora.e2m1_value(c) == want, c


def _e2m1_expected(v):
    """Nearest E2M1 code from the midpoints of the published value set, ties to
    the even code, |v| >= 6 -> 6, sign kept; formulated with thresholds, not
    with the oracle's search."""
    vals = _gold("e2m1_values.json")["values"]
    if math.isnan(v):
        return 0
    sign = 8 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    code = 0
    for c in range(1, 8):
        mid = (vals[c - 1] + vals[c]) / 2.0
        if a > mid or (a == mid and c % 2 == 0):
            code = c
    return sign | code


def test_e2m1_encode_near_every_threshold(ora):
    vals = _gold("e2m1_values.json")["values"]
    pts = set()
    for c in range(8):
        for m in [vals[c]] + ([(vals[c - 1] + vals[c]) / 2] if c else []):
            b = int(np.float32(m).view(np.uint32))
            for d in range(-3, 4):
                if b + d >= 0:
                    pts.add(b + d)
    pts |= {0, 0x7F800000, 0x7F7FFFFF, 0x00000001, 0x007FFFFF, 0x00800000,
            int(np.float32(5.9999995).view(np.uint32)), int(np.float32(7.0).view(np.uint32))}
    for b in sorted(pts):
        for sb in (0, 0x80000000):
            v = float(f32(b | sb))
            assert ora.e2m1_encode(v) == _e2m1_expected(v), hex(b | sb)
    assert ora.e2m1_encode(float("nan")) == 0
    assert ora.e2m1_encode(-0.0) == 0x8
    assert ora.e2m1_encode(float("inf")) == 7 and ora.e2m1_encode(float("-inf")) == 15


def test_e2m1_encode_random_sample(ora):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32)
    small = (rng.random(4000) * 14 - 7).astype(np.float32).view(np.uint32)
    for b in np.concatenate([bits, small]):
        v = float(f32(b))
        assert ora.e2m1_encode(v) == _e2m1_expected(v), hex(int(b))


def test_every_bf16_through_element_quantizer_at_unit_scale(ora):
    """All 65,536 bf16 inputs with sf = 1.0 (0x38) and s_g = 1, so d = 1 and the
    quotient is the value itself; every E2M1 midpoint is a bf16 value."""
    for h in range(65536):
        v = float(bf16_to_f32_np(h))
        assert ora.element_code(h, 0x38, 1.0) == _e2m1_expected(v), hex(h)


def test_element_code_zero_when_sf_zero(ora):
    for h in (0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x8000):
        assert ora.element_code(h, 0, 1.0) == 0


# --------------------------------------------------------------------------
# E4M3
# --------------------------------------------------------------------------
def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_torch_and_spec(ora):
    tv = _torch_e4m3_values()
    for c in range(256):
        v = ora.e4m3_value(c)
        if math.isnan(tv[c]):
            assert math.isnan(v), hex(c)
        else:
            assert v == tv[c], hex(c)
    pts = _gold("e4m3_points.json")
    for k, want in pts["points"].items():
        assert ora.e4m3_value(int(k, 16)) == want
    for k in pts["nan_codes"]:
        assert math.isnan(ora.e4m3_value(int(k, 16)))


def _e4m3_probe_points():
    """Structured f32 points covering every rounding case of a 3-bit mantissa:
    all exponents from 2^-12 to 2^9, all 5-bit mantissa prefixes, and low
    ('sticky') bit patterns 0, 1, mid and all-ones; plus random points."""
    pts = []
    for e in range(127 - 12, 127 + 10):
        for top in range(32):
            for low in (0, 1, 1 << 17, (1 << 18) - 1):
                pts.append((e << 23) | (top << 18) | low)
    rng = np.random.default_rng(7)
    r = (rng.random(20000) * 470.0).astype(np.float32).view(np.uint32)
    r2 = (2.0 ** rng.uniform(-14, 9, 20000)).astype(np.float32).view(np.uint32)
    return np.concatenate([np.array(pts, np.uint32), r, r2])


def test_e4m3_encode_matches_torch_cast_below_464(ora):
    """torch's float -> float8_e4m3fn cast rounds to nearest-even; for t < 464
    it never saturates, so it must equal the oracle's encoder exactly."""
    bits = _e4m3_probe_points()
    t = f32(bits)
    t = t[(t >= 0) & (t < 464)]
    want = torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i in range(t.size):
        got = ora.e4m3_encode(float(t[i]))
        assert got == want[i], (float(t[i]), hex(got), hex(int(want[i])))


def test_e4m3_encode_all_bf16_values(ora):
    """Every non-negative finite bf16 value below 464 vs torch's cast."""
    h = np.arange(0, 0x7F80, dtype=np.uint32)
    t = bf16_to_f32_np(h)
    t = t[t < 464]
    want = torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([ora.e4m3_encode(float(v)) for v in t], np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_saturation_and_specials(ora):
    assert ora.e4m3_encode(448.0) == 0x7E
    assert ora.e4m3_encode(463.99997) == 0x7E
    assert ora.e4m3_encode(464.0) == 0x7E
    assert ora.e4m3_encode(1e30) == 0x7E
    assert ora.e4m3_encode(float("inf")) == 0x7E
    assert ora.e4m3_encode(float("nan")) == 0x7F
    assert ora.e4m3_encode(0.0) == 0x00
    assert ora.e4m3_encode(2.0 ** -10) == 0x00          # tie between 0 and 2^-9 -> even code 0
    assert ora.e4m3_encode(1.5 * 2.0 ** -10) == 0x01
    assert ora.e4m3_encode(3 * 2.0 ** -10) == 0x02      # tie between codes 1 and 2 -> even
    assert ora.e4m3_encode(5 * 2.0 ** -10) == 0x02      # tie between codes 2 and 3 -> even


# --------------------------------------------------------------------------
# BF16 rounding
# --------------------------------------------------------------------------
def _bf16_probe_bits():
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    pts = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(3)
    return np.concatenate([pts, rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)])


def test_f32_to_bf16_matches_torch(ora):
    bits = _bf16_probe_bits()
    x = torch.from_numpy(f32(bits).copy())
    want = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    L = ora.lib()
    got = np.fromiter((L.ora_f32_to_bf16(float(v)) for v in f32(bits)), np.uint16, bits.size)
    nan = np.isnan(f32(bits))
    assert np.array_equal(got[~nan], want[~nan])
    # NaN: quiet NaN with the sign kept
    assert np.all((got[nan] & 0x7FC0) == 0x7FC0)
    assert np.array_equal(got[nan] >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_f32_to_bf16_exact_rational_rounding(ora):
    """Closed form: the chosen bf16 is one of the two neighbours and no farther
    from the input than the other; at an exact tie the mantissa is even."""
    from fractions import Fraction

    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F7F0000, 3000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, (np.arange(0, 0x7F7F, 97, dtype=np.uint32) << 16) | 0x8000])
    for b in bits:
        v = float(f32(b))
        h = ora.f32_to_bf16(v)
        lo = int(b) >> 16
        cand = (lo, lo + 1)
        assert h in cand
        fv = Fraction(v)
        d = [abs(fv - Fraction(float(bf16_to_f32_np(c)))) for c in cand]
        mine = d[cand.index(h)]
        assert mine <= min(d)
        if d[0] == d[1]:
            assert h % 2 == 0


# --------------------------------------------------------------------------
# Modulation: exact BF16 op order
# --------------------------------------------------------------------------
def _torch_modulate(x, scale, shift):
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    st = torch.from_numpy(scale.view(np.int16)).view(torch.bfloat16)
    ht = torch.from_numpy(shift.view(np.int16)).view(torch.bfloat16)
    y = (xt * (st + 1)) + ht
    return y.view(torch.int16).numpy().view(np.uint16)


def _random_bf16(rng, n, spread=True):
    if spread:
        return rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    return (torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def test_modulation_matches_torch_bf16_ops(ora):
    """torch computes each bf16 op in binary32 and rounds to bf16: the same
    three roundings, in the order (x * (scale + 1)) + shift."""
    rng = np.random.default_rng(5)
    n = 60000
    cases = [
        (_random_bf16(rng, n, False), _random_bf16(rng, n, False), _random_bf16(rng, n, False)),
        (_random_bf16(rng, n), _random_bf16(rng, n), _random_bf16(rng, n)),
    ]
    for x, sc, sh in cases:
        finite = ~np.isnan(bf16_to_f32_np(x)) & ~np.isnan(bf16_to_f32_np(sc)) & ~np.isnan(bf16_to_f32_np(sh))
        want = _torch_modulate(x, sc, sh)
        L = ora.lib()
        got = np.fromiter((L.ora_modulate(int(a), int(b), int(c)) for a, b, c in zip(x, sc, sh)), np.uint16, n)
        wn = np.isnan(bf16_to_f32_np(want))
        ok = (got == want) | (wn & np.isnan(bf16_to_f32_np(got)))
        assert ok[finite].all(), np.flatnonzero(~ok & finite)[:5]


def test_modulation_order_is_discriminated(ora):
    """Alternative readings (one rounding for the whole expression, scale+1 not
    rounded, an FMA) give different bytes on some inputs; the oracle equals
    the three-rounding reading on all of them."""
    rng = np.random.default_rng(9)
    n = 40000
    x, sc, sh = _random_bf16(rng, n, False), _random_bf16(rng, n, False), _random_bf16(rng, n, False)
    xf, sf, hf = (bf16_to_f32_np(a).astype(np.float64) for a in (x, sc, sh))
    to_bf = lambda v: torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    single = to_bf(xf * (sf + 1.0) + hf)                             # exact, one rounding
    s1 = np.float32(sf + 1.0).astype(np.float64)                     # scale+1 in f32, not bf16
    unrounded_s = to_bf(bf16_to_f32_np(to_bf(np.float32(xf * s1))).astype(np.float64) + hf)
    L = ora.lib()
    got = np.fromiter((L.ora_modulate(int(a), int(b), int(c)) for a, b, c in zip(x, sc, sh)), np.uint16, n)
    assert np.count_nonzero(got != single) > 0
    assert np.count_nonzero(got != unrounded_s) > 0
    assert np.array_equal(got, _torch_modulate(x, sc, sh))


def test_identity_modulation_is_exact(ora):
    """scale = +0 and shift = -0 give y = x bit-exactly for every bf16 x that
    is not NaN (used to prepack weights through the modulation producer)."""
    L = ora.lib()
    for h in range(65536):
        if (h & 0x7FFF) > 0x7F80:
            continue
        assert L.ora_modulate(h, 0x0000, 0x8000) == h, hex(h)


# --------------------------------------------------------------------------
# SwiGLU: correctly rounded exp and the silu chain
# --------------------------------------------------------------------------
def _cr_float32(mpf_val, mp):
    """Correctly rounded binary32 of a multiprecision value."""
    if mpf_val >= (2 - mp.mpf(2) ** -24) * mp.mpf(2) ** 127:  # rounds past the largest finite
        return np.float32(np.inf)
    f0 = np.float32(float(mpf_val))
    best, bd = f0, None
    for c in (np.nextafter(f0, np.float32(-np.inf)), f0, np.nextafter(f0, np.float32(np.inf))):
        if not np.isfinite(c):
            continue
        d = abs(mp.mpf(float(c)) - mpf_val)
        if bd is None or d < bd or (d == bd and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best, bd = c, d
    return best


@pytest.mark.slow
def test_exp_neg_is_correctly_rounded_for_every_bf16(ora):
    mp = pytest.importorskip("mpmath")
    mp.mp.prec = 200
    L = ora.lib()
    for h in range(65536):
        g = float(bf16_to_f32_np(h))
        if not math.isfinite(g):
            continue
        got = np.float32(L.ora_exp_neg(h))
        want = _cr_float32(mp.exp(-mp.mpf(g)), mp)
        assert got == want or (np.isinf(got) and np.isinf(want)), (hex(h), got, want)


def test_silu_bf16_against_exact_silu(ora):
    """For every finite bf16 gate, the binary32 chain rounded to bf16 equals the
    exact silu rounded to bf16, except (a) where exp(-g) overflows binary32
    (g < -88.72: the chain gives -0) and (b) where the exact silu lies within
    2^-20 relative of a bf16 rounding midpoint (double-rounding window)."""
    mp = pytest.importorskip("mpmath")
    mp.mp.prec = 80
    L = ora.lib()
    exceptions = 0
    for h in range(0, 65536, 3):
        g = float(bf16_to_f32_np(h))
        if not math.isfinite(g):
            continue
        got = L.ora_silu_bf16(h)
        if g < -88.72:
            assert got in (0x8000, 0x0000) or got & 0x8000, hex(h)
            continue
        gm = mp.mpf(g)
        s = gm / (1 + mp.exp(-gm))
        sf = float(s)
        want = int(torch.tensor([sf], dtype=torch.float64).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        if got != want:
            lo = float(bf16_to_f32_np(min(got, want) & 0x7FFF))
            hi = float(bf16_to_f32_np(max(got, want) & 0x7FFF))
            mid = (lo + hi) / 2
            assert abs(abs(sf) - mid) <= 2.0 ** -20 * abs(sf), (hex(h), hex(got), hex(want))
            exceptions += 1
    assert exceptions < 20


def test_swiglu_is_silu_times_up_rounded(ora):
    """h = bf16(silu_bf16(g) * up): the product step against torch's bf16 multiply."""
    L = ora.lib()
    rng = np.random.default_rng(2)
    g = _random_bf16(rng, 3000, False)
    u = _random_bf16(rng, 3000, False)
    sb = np.array([L.ora_silu_bf16(int(a)) for a in g], np.uint16)
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
    want = (tb(sb) * tb(u)).view(torch.int16).numpy().view(np.uint16)
    got = np.array([L.ora_swiglu(int(a), int(b)) for a, b in zip(g, u)], np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# Scales
# --------------------------------------------------------------------------
def test_tensor_scale(ora):
    assert ora.tensor_scale(0.0) == 1.0
    assert ora.tensor_scale(2688.0) == 1.0
    assert ora.tensor_scale(6.0) == float(np.float32(6.0) / np.float32(2688.0))
    assert math.isinf(ora.tensor_scale(float("inf")))
    assert math.isnan(ora.tensor_scale(float("nan")))


def test_global_block_invariants_for_every_bf16_amax(ora):
    """Closed form over all 32,640 positive finite bf16 amax: the block holding
    the global maximum gets sf = 448 (0x7E) and the maximum itself encodes as
    6 (code 7); the block-scale argument never reaches 464, so saturation is
    never needed for finite input."""
    L = ora.lib()
    for h in range(1, 0x7F80):
        amax = float(bf16_to_f32_np(h))
        s_g = np.float32(L.ora_tensor_scale(amax))
        t = np.float32(np.float32(np.float32(amax) / np.float32(6.0)) / s_g)
        assert t < 464.0
        assert L.ora_block_scale(amax, float(s_g)) == 0x7E, hex(h)
        assert L.ora_element_code(h, 0x7E, float(s_g)) == 7, hex(h)
        assert L.ora_element_code(h | 0x8000, 0x7E, float(s_g)) == 15, hex(h)


def test_e2m1_times_e4m3_products_are_exact_in_bf16(ora):
    """Every product of a finite E2M1 value and a finite E4M3 value is exactly
    representable in bf16 (and in fp16): 8 x 127 non-negative cases."""
    n = 0
    for c in range(8):
        for s in range(0x7F):
            p = ora.e2m1_value(c) * ora.e4m3_value(s)
            b = torch.tensor([p], dtype=torch.float64)
            assert b.to(torch.bfloat16).to(torch.float64).item() == p
            assert b.to(torch.float16).to(torch.float64).item() == p
            n += 1
    assert n == 1016


# --------------------------------------------------------------------------
# Exact residual epilogue: out = bf16(residual + bf16(gate * o))
# --------------------------------------------------------------------------
def _torch_gate_residual(o, g, r):
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)  # noqa: E731
    return (to(r) + to(g) * to(o)).view(torch.int16).numpy().view(np.uint16)


def test_gate_residual_matches_torch_bf16_ops(ora):
    """torch evaluates residual + gate * o on bf16 tensors as two binary32
    operations, each rounded to bf16: the oracle's step, bit for bit (NaN
    results compared as NaN)."""
    rng = np.random.default_rng(21)
    n = 60000
    L = ora.lib()
    for spread in (False, True):
        o, g, r = (_random_bf16(rng, n, spread) for _ in range(3))
        want = _torch_gate_residual(o, g, r)
        got = np.fromiter((L.ora_gate_residual(int(a), int(b), int(c)) for a, b, c in zip(o, g, r)), np.uint16, n)
        wn = np.isnan(bf16_to_f32_np(want))
        ok = (got == want) | (wn & np.isnan(bf16_to_f32_np(got)))
        assert ok.all(), np.flatnonzero(~ok)[:5]


def test_gate_residual_rounds_the_product_first(ora):
    """One rounding of the whole residual + gate * o gives different bytes on
    some inputs; the oracle keeps the bf16 rounding of the product."""
    rng = np.random.default_rng(22)
    n = 40000
    o, g, r = (_random_bf16(rng, n, False) for _ in range(3))
    of, gf, rf = (bf16_to_f32_np(a).astype(np.float64) for a in (o, g, r))
    single = (torch.from_numpy(rf + gf * of).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    L = ora.lib()
    got = np.fromiter((L.ora_gate_residual(int(a), int(b), int(c)) for a, b, c in zip(o, g, r)), np.uint16, n)
    assert np.count_nonzero(got != single) > 0
    assert np.array_equal(got, _torch_gate_residual(o, g, r))


def test_unit_gate_zero_residual_is_identity(ora):
    """gate = 1 and residual = -0 return o bit-exactly for every non-NaN bf16."""
    L = ora.lib()
    for h in range(65536):
        if (h & 0x7FFF) > 0x7F80:
            continue
        assert L.ora_gate_residual(h, 0x3F80, 0x8000) == h, hex(h)
