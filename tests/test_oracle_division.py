"""Pins for the oracle's three division steps (CPU only).

"NVFP4 Streaming Design", Numerical Constraint: the tensor's exact maximum
magnitude gives one FP32 tensor scale, each 16 values get an E4M3 scale, and
the E2M1 codes come from both scales.  The quantizer fixed for this path reads
those steps as correctly rounded binary32 operations:

    s_g = RN(amax / 2688)                      (2688 = 6 * 448; 1 when amax = 0)
    sf  = E4M3(RN(RN(a16 / 6) / s_g))
    q   = E2M1(RN(y / RN(float(sf) * s_g)))

Each pin below recomputes a step from exact rational arithmetic (integers,
rounded once into binary32 by ``_exact``), encodes with torch's float8 cast or
with the threshold encoder of the published E2M1 value set, and compares every
case with the oracle.  Each also shows that the plausible other readings of the
same step (a different grouping of the divisions, one rounding instead of two,
a reciprocal) give different bytes on the tested set, so a swapped reading in
the oracle would fail the pin.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests import _exact as X

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16_f32(h):
    return (np.asarray(h, np.uint32) << 16).view(np.float32)


def e4m3_cast(t: np.ndarray) -> np.ndarray:
    """torch's nearest-even binary32 -> float8_e4m3fn cast, as code bytes."""
    return torch.from_numpy(np.ascontiguousarray(t, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_values() -> np.ndarray:
    """The 256 E4M3FN code values from torch's decode (NaN for 0x7F / 0xFF)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def e2m1_threshold_encode(q: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code of |q| >= 0 from the midpoints of the published value
    set: each midpoint passed adds one code, a value on a midpoint passes it
    only towards the even code; 6 and beyond saturate to code 7."""
    with open(os.path.join(GOLD, "e2m1_values.json")) as f:
        vals = json.load(f)["values"]
    a = np.asarray(q, np.float64)
    code = np.zeros(a.shape, np.uint8)
    for c in range(1, 8):
        mid = (vals[c - 1] + vals[c]) / 2.0
        code += ((a > mid) | ((a == mid) & (c % 2 == 0))).astype(np.uint8)
    return code


# --------------------------------------------------------------------------
# the exact-rounding helper itself, against Python's Fraction
# --------------------------------------------------------------------------
def test_exact_rounding_helper_matches_fractions():
    rng = np.random.default_rng(31)
    a = rng.integers(1, 0x7F800000, 4000, dtype=np.int64).astype(np.uint32).view(np.float32)
    b = rng.integers(1, 0x7F800000, 4000, dtype=np.int64).astype(np.uint32).view(np.float32)
    # add subnormal, overflow and exact-tie corners
    a = np.concatenate([a, np.float32([1.0, 3.0, 2.0 ** -149, 2.0 ** -126, 3.0e38, 1.5 * 2.0 ** -140])])
    b = np.concatenate([b, np.float32([3.0, 2.0 ** 24 + 2, 2.0, 3.0, 1e-3, 2.0 ** 10])])
    q = X.div32(a, b)
    p = X.mul32(a, b)
    for i in range(a.size):
        fa, fb = Fraction(float(a[i])), Fraction(float(b[i]))
        assert q[i].view(np.uint32) == X.rn32_fraction(fa / fb).view(np.uint32), (a[i], b[i])
        assert p[i].view(np.uint32) == X.rn32_fraction(fa * fb).view(np.uint32), (a[i], b[i])
    # ties: 1 + 2^-24 is halfway between 1 and 1 + 2^-23 -> even (1);
    # 1 + 3 * 2^-24 is halfway between 1 + 2^-23 and 1 + 2^-22 -> even (1 + 2^-22)
    t = X.round_ratio(np.int64([(1 << 24) + 1, (1 << 24) + 3]), 1, -24)
    assert t[0] == np.float32(1.0) and t[1] == np.float32(1.0 + 2.0 ** -22)


# --------------------------------------------------------------------------
# tensor scale: s_g = RN(amax / 2688)
# --------------------------------------------------------------------------
def test_tensor_scale_every_bf16_amax(ora):
    L = ora.lib()
    h = np.arange(1, 0x7F80, dtype=np.uint32)        # every positive finite bf16
    amax = bf16_f32(h)
    want = X.div32_int(amax, 2688)
    got = np.fromiter((L.ora_tensor_scale(float(v)) for v in amax), np.float32, amax.size)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), np.flatnonzero(got != want)[:5]
    assert L.ora_tensor_scale(0.0) == 1.0
    # other readings of "amax / (6 * 448)" give different scales on this set
    two_step = X.div32_int(X.div32_int(amax, 6), 448)
    recip = X.mul32(amax, X.div32_int(np.float32([1.0]), 2688))
    assert np.count_nonzero(two_step != want) > 1000
    assert np.count_nonzero(recip != want) > 1000


# --------------------------------------------------------------------------
# block scale: sf = E4M3(RN(RN(a16 / 6) / s_g))
# --------------------------------------------------------------------------
def _tensor_scale_amaxes():
    """130 tensor maxima spread over every bf16 binade (subnormal to the
    largest finite), plus the round values that matter for the workloads."""
    step = np.arange(1, 0x7F80, 251, dtype=np.uint32)
    extra = np.array([0x3F80, 0x40C0, 0x4396, 0x4528, 0x4170, 0x7F7F, 0x0001, 0x0080, 0x3A83], np.uint32)
    return np.unique(np.concatenate([step, extra]))


def test_block_scale_every_a16_at_many_tensor_scales(ora):
    """For each tensor maximum, every bf16 block maximum a16 from 0 to that
    maximum (the only ones a block can have) through the block-scale step."""
    amaxes = _tensor_scale_amaxes()
    assert amaxes.size >= 130
    total = 0
    alt_div_by_product = 0
    alt_single_rounding = 0
    for hm in amaxes:
        amax = bf16_f32(hm)
        s_g = X.div32_int(np.float32([amax]), 2688)[0]
        a16_bits = np.arange(0, hm + 1, dtype=np.uint32)
        a16 = bf16_f32(a16_bits)
        t = X.div32(X.div32_int(a16, 6), np.full(a16.shape, s_g, np.float32))
        assert np.all(t < 464.0)                       # torch's cast needs no saturation here
        want = e4m3_cast(t)
        got = ora.block_scale_batch(a16_bits.astype(np.uint16), float(s_g))
        assert np.array_equal(got, want), (hex(int(hm)), np.flatnonzero(got != want)[:5])
        total += a16.size
        # a16 / RN(6 s_g), and a16 / (6 s_g) rounded once
        six_sg = X.mul32(np.float32([6.0]), np.float32([s_g]))
        alt1 = e4m3_cast(X.div32(a16, np.full(a16.shape, six_sg[0], np.float32)))
        sm, se = X.decompose(np.float32([s_g]))
        am, ae = X.decompose(a16)
        alt2 = e4m3_cast(X.round_ratio(am, 6 * sm[0], ae - se[0]))
        alt_div_by_product += int(np.count_nonzero(alt1 != want))
        alt_single_rounding += int(np.count_nonzero(alt2 != want))
    assert total > 2_000_000
    assert alt_div_by_product > 0, "grouping a16 / (6 s_g) is not discriminated"
    assert alt_single_rounding > 0, "a single rounding of a16 / (6 s_g) is not discriminated"


# --------------------------------------------------------------------------
# element code: q = E2M1(RN(y / RN(float(sf) * s_g)))
# --------------------------------------------------------------------------
def _element_code_reference(y_bits, sf_val, s_g, grouping="spec"):
    """Codes for every y in y_bits at one scale code value and tensor scale,
    by exact rational arithmetic; grouping selects an alternative reading."""
    y = bf16_f32(y_bits)
    sign = ((y_bits >> 15) & 1).astype(np.uint8) * 8
    mag_bits = y_bits & 0x7FFF
    finite = mag_bits < 0x7F80
    nan = mag_bits > 0x7F80
    ymag = np.abs(np.where(finite, y, np.float32(0.0))).astype(np.float32)
    sfa = np.float32([sf_val])
    sga = np.float32([s_g])
    if grouping == "spec":
        d = X.mul32(sfa, sga)[0]
        q = X.div32(ymag, np.full(ymag.shape, d, np.float32)) if d > 0 else None
    elif grouping == "y_over_sf_then_sg":
        d = np.float32(1.0)
        first = X.div32(ymag, np.full(ymag.shape, sfa[0], np.float32))
        big = ~np.isfinite(first)                        # y / sf overflowed: the quotient stays infinite
        q = X.div32(np.where(big, np.float32(0.0), first), np.full(ymag.shape, sga[0], np.float32))
        q = np.where(big, np.float32(np.inf), q)
    elif grouping == "single_rounding":
        d = np.float32(1.0)
        fm, fe = X.decompose(sfa)
        gm, ge = X.decompose(sga)
        ym, ye = X.decompose(ymag)
        q = X.round_ratio(ym, fm[0] * gm[0], ye - fe[0] - ge[0])
    elif grouping == "reciprocal":
        d = X.mul32(sfa, sga)[0]
        r = X.div32(np.float32([1.0]), np.float32([d]))
        if not np.isfinite(r[0]):
            return None                                  # no finite reciprocal to compare with
        q = X.mul32(ymag, np.full(ymag.shape, r[0], np.float32))
    else:
        raise ValueError(grouping)
    if d > 0:
        mag = e2m1_threshold_encode(q)
        mag = np.where(finite, mag, 7)                  # an infinite y gives an infinite quotient: 6
    else:
        # d underflowed to 0: y / 0 is infinite (code 6) except 0 / 0 (NaN, code 0)
        mag = np.where(ymag > 0, 7, 0).astype(np.uint8)
        mag = np.where(finite, mag, 7)
        code = (sign | mag).astype(np.uint8)
        code[(ymag == 0) & finite] = 0
        code[nan] = 0
        return code
    code = (sign | mag).astype(np.uint8)
    code[nan] = 0
    return code


ELEMENT_TENSOR_SCALES = [0x3F80, 0x40C0, 0x4396, 0x4170, 0x3A83, 0x7F7F, 0x0001]


@pytest.mark.parametrize("amax_bits", ELEMENT_TENSOR_SCALES, ids=lambda h: f"amax{h:04x}")
def test_element_code_every_y_every_scale_code(ora, amax_bits):
    """All 65,536 bf16 y against all 126 finite nonzero scale codes at one
    tensor scale (from the tensor maximum amax_bits)."""
    s_g = X.div32_int(bf16_f32(np.uint32([amax_bits])), 2688)[0]
    y_bits = np.arange(65536, dtype=np.uint32)
    sfv = e4m3_values()
    for sf in range(1, 0x7F):
        want = _element_code_reference(y_bits, sfv[sf], s_g)
        got = ora.element_code_batch(y_bits.astype(np.uint16), np.full(65536, sf, np.uint8), float(s_g))
        assert np.array_equal(got, want), (hex(sf), np.flatnonzero(got != want)[:5])
    # sf = 0 packs to zero for every y
    got0 = ora.element_code_batch(y_bits.astype(np.uint16), np.zeros(65536, np.uint8), float(s_g))
    assert not got0.any()


def test_element_code_other_readings_are_discriminated(ora):
    """The groupings y / sf / s_g, one rounding of y / (sf s_g), and y times a
    rounded reciprocal each change some codes inside the exhaustive pin's
    domain (at the tensor maximum 6.0 already from scale codes 3-5 on), so the
    pin separates each of them from the reading taken.  The scan stops once
    all three are seen."""
    y_bits = np.arange(65536, dtype=np.uint32)
    sfv = e4m3_values()
    seen = set()
    for amax_bits in [0x40C0] + [h for h in ELEMENT_TENSOR_SCALES if h != 0x40C0]:
        s_g = X.div32_int(bf16_f32(np.uint32([amax_bits])), 2688)[0]
        if X.mul32(np.float32([2.0 ** -9]), np.float32([s_g]))[0] == 0:
            continue                                     # alternatives need a nonzero divisor
        for sf in range(1, 0x7F):
            want = _element_code_reference(y_bits, sfv[sf], s_g)
            for g in ("y_over_sf_then_sg", "single_rounding", "reciprocal"):
                if g in seen:
                    continue
                alt = _element_code_reference(y_bits, sfv[sf], s_g, g)
                if alt is not None and np.count_nonzero(alt != want):
                    seen.add(g)
            if len(seen) == 3:
                return
    pytest.fail(f"readings not discriminated: {sorted({'y_over_sf_then_sg', 'single_rounding', 'reciprocal'} - seen)}")
