"""Each device step of the producer against the oracle over its whole (or a
structured covering) input domain, through the single-step C entry points."""
import numpy as np
import pytest
import torch

import oracle
from tests import _par
from tests.gpu_util import device, first_mismatch, host, to_dev, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import nvfp4_activation_quantization_segment_amd as pkg

    device()
    return pkg


def _sync():
    torch.cuda.synchronize()


def bf16_values(h):
    return (np.asarray(h, np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
def test_step_modulate_random_and_ties(m):
    rng = np.random.default_rng(21)
    n = 1 << 21
    x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    sc = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    sh = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    # normal-range values, where BF16 ties in the product and sum are frequent
    xn = (torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)
          .view(torch.int16).numpy().view(np.uint16))
    scn = (torch.from_numpy((0.1 * rng.standard_normal(n)).astype(np.float32)).to(torch.bfloat16)
           .view(torch.int16).numpy().view(np.uint16))
    shn = (torch.from_numpy((0.1 * rng.standard_normal(n)).astype(np.float32)).to(torch.bfloat16)
           .view(torch.int16).numpy().view(np.uint16))
    for a, b, c in ((x, sc, sh), (xn, scn, shn)):
        finite = ((a & 0x7FFF) <= 0x7F80) & ((b & 0x7FFF) <= 0x7F80) & ((c & 0x7FFF) <= 0x7F80)
        want = _par.batch(oracle.modulate_batch, n, a, b, c)
        y = torch.empty(n, dtype=torch.int16, device=device())
        m.nvfp4_step_modulate(to_dev_u16(a), to_dev_u16(b), to_dev_u16(c), y, n)
        _sync()
        got = host(y).view(np.uint16)
        nan_w = (want & 0x7FFF) > 0x7F80
        nan_g = (got & 0x7FFF) > 0x7F80
        ok = (got == want) | (nan_w & nan_g)
        assert ok[finite].all(), first_mismatch(got[finite], want[finite])


def test_step_silu_every_bf16_gate(m):
    """silu_bf16 over all 65,536 gates (up = 1.0, so h = bf16(silu(g)))."""
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    u = np.full(65536, 0x3F80, np.uint16)
    want = oracle.swiglu_batch(g, u)
    h = torch.empty(65536, dtype=torch.int16, device=device())
    m.nvfp4_step_swiglu(to_dev_u16(g), to_dev_u16(u), h, 65536)
    _sync()
    got = host(h).view(np.uint16)
    finite = (g & 0x7FFF) < 0x7F80
    assert np.array_equal(got[finite], want[finite]), first_mismatch(got[finite], want[finite])


def test_step_swiglu_random(m):
    rng = np.random.default_rng(22)
    n = 1 << 20
    g = (torch.from_numpy((3 * rng.standard_normal(n)).astype(np.float32)).to(torch.bfloat16)
         .view(torch.int16).numpy().view(np.uint16))
    u = (torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)
         .view(torch.int16).numpy().view(np.uint16))
    want = _par.batch(oracle.swiglu_batch, n, g, u)
    h = torch.empty(n, dtype=torch.int16, device=device())
    m.nvfp4_step_swiglu(to_dev_u16(g), to_dev_u16(u), h, n)
    _sync()
    got = host(h).view(np.uint16)
    assert np.array_equal(got, want), first_mismatch(got, want)


# tensor scales to test: s_g of bf16 maxima across the whole range, including
# the ones outside the Markstein fast range
def _scales():
    amax_bits = [0x0001, 0x0080, 0x0F00, 0x1234, 0x2A00, 0x3000, 0x3380, 0x3A00, 0x3C00, 0x3E4C, 0x3F80, 0x4000,
                 0x4040, 0x40C0, 0x4110, 0x4300, 0x4396, 0x4500, 0x4780, 0x5000, 0x6000, 0x7000, 0x7F00, 0x7F7F]
    rng = np.random.default_rng(23)
    amax_bits += list(rng.integers(0x0080, 0x7F7F, 12))
    return [oracle.tensor_scale(float(bf16_values(b))) for b in amax_bits]


def test_step_block_scale_all_maxima(m):
    a16 = np.arange(0, 0x7F81, dtype=np.uint32).astype(np.uint16)  # every finite magnitude, and +inf
    sg_dev = torch.empty(1, dtype=torch.float32, device=device())
    sf = torch.empty(a16.size, dtype=torch.uint8, device=device())
    a_dev = to_dev_u16(a16)
    for s_g in _scales():
        sg_dev.fill_(s_g)
        m.nvfp4_step_block_scale(a_dev, sg_dev, sf, a16.size)
        _sync()
        got = host(sf)
        want = _par.batch(lambda a: oracle.block_scale_batch(a, s_g), a16.size, a16)
        assert np.array_equal(got, want), (s_g, first_mismatch(got, want))


def test_step_element_code_all_values(m):
    """Every bf16 y against every E4M3 block scale (0, all finite codes and the
    NaN code) for tensor scales across the range, and for maxima whose 8-bit
    mantissa shares a factor 3 or 7 with 2688 = 2^7 * 3 * 7 (168, 210, 252,
    140; s_g = 1 at 2688), where s_g is a short or short-period binary
    fraction and quotients fall exactly on or next to E2M1 midpoints."""
    y = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    y = y[(y & 0x7FFF) <= 0x7F80]  # finite values and +-inf
    sfs = np.arange(0, 0x80, dtype=np.uint8)
    Y = np.tile(y, sfs.size)
    S = np.repeat(sfs, y.size)
    y_dev, s_dev = to_dev_u16(Y), to_dev(S)
    code = torch.empty(Y.size, dtype=torch.uint8, device=device())
    sg_dev = torch.empty(1, dtype=torch.float32, device=device())
    structured = [0x4528, 0x3FD2, 0x27D2, 0x4128, 0x31FC, 0x2E8C]
    for s_g in _scales() + [oracle.tensor_scale(float(bf16_values(b))) for b in structured]:
        sg_dev.fill_(s_g)
        m.nvfp4_step_element_code(y_dev, s_dev, sg_dev, code, Y.size)
        _sync()
        got = host(code)
        want = _par.batch(lambda a, b: oracle.element_code_batch(a, b, s_g), Y.size, Y, S)
        assert np.array_equal(got, want), (s_g, first_mismatch(got, want))


def _f32_cover(lo_exp, hi_exp, rng, nrand):
    """Every binary32 exponent in [lo_exp, hi_exp] x all 8-bit mantissa prefixes x
    low patterns {0, 1, half, all ones}, both signs; plus random values."""
    e = np.arange(lo_exp + 127, hi_exp + 128, dtype=np.uint32)
    top = np.arange(256, dtype=np.uint32) << 15
    low = np.array([0, 1, 1 << 14, (1 << 15) - 1], np.uint32)
    bits = ((e[:, None, None] << 23) | top[None, :, None] | low[None, None, :]).ravel()
    bits = np.concatenate([bits, bits | 0x80000000, np.array([0, 0x80000000, 1, 0x80000001, 0x7F800000,
                                                               0xFF800000, 0x7F7FFFFF], np.uint32)])
    r = rng.integers(0, 2**32, nrand, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([bits, r]).view(np.float32)


def test_step_e2m1_conversion(m):
    rng = np.random.default_rng(24)
    v = _f32_cover(-30, 4, rng, 1 << 20)
    small = (rng.random(1 << 20) * 14 - 7).astype(np.float32)
    thr = []
    for t in (0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0):
        b = np.float32(t).view(np.uint32)
        thr.append((b + np.arange(-64, 65)).astype(np.uint32))
    tb = np.concatenate(thr)
    v = np.concatenate([v, small, tb.view(np.float32), (tb | 0x80000000).view(np.float32)])
    v = v[~np.isnan(v)]
    code = torch.empty(v.size, dtype=torch.uint8, device=device())
    m.nvfp4_step_e2m1(to_dev(v), code, v.size)
    _sync()
    got = host(code)
    want = _par.batch(oracle.e2m1_batch, v.size, v)
    assert np.array_equal(got, want), first_mismatch(got, want)


def test_step_e4m3_conversion(m):
    rng = np.random.default_rng(25)
    v = _f32_cover(-30, 9, rng, 0)
    v = np.abs(v)
    v = np.concatenate([v, (rng.random(1 << 20) * 470).astype(np.float32),
                        bf16_values(np.arange(0, 0x7F81, dtype=np.uint32)),
                        np.array([np.inf, 448.0, 464.0, 465.0, 2.0 ** -10, 3 * 2.0 ** -10], np.float32)])
    code = torch.empty(v.size, dtype=torch.uint8, device=device())
    m.nvfp4_step_e4m3(to_dev(v), code, v.size)
    _sync()
    got = host(code)
    want = _par.batch(oracle.e4m3_batch, v.size, v)
    assert np.array_equal(got, want), first_mismatch(got, want)
    nan = torch.full((4,), float("nan"), device=device())
    c4 = torch.empty(4, dtype=torch.uint8, device=device())
    m.nvfp4_step_e4m3(nan, c4, 4)
    _sync()
    assert (host(c4) == 0x7F).all()
