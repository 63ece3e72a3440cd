"""Pins for the oracle's tensor passes and GEMM reference (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def tb(a):
    """uint16 numpy bf16 bits -> torch bf16 tensor (shares memory)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def nb(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def torch_modulated(x, row_start, shift, scale):
    """y via torch bf16 ops with per-row gathered segment rows (library check)."""
    M = x.shape[0]
    seg_of_row = np.searchsorted(np.asarray(row_start[1:]), np.arange(M), side="right")
    sh = tb(shift)[torch.from_numpy(seg_of_row)]
    sc = tb(scale)[torch.from_numpy(seg_of_row)]
    return nb((tb(x) * (sc + 1)) + sh)


def small_case(seed, M=200, D=96, segs=(0, 37, 150, 200)):
    rng = np.random.default_rng(seed)
    x = nb(torch.from_numpy(rng.standard_normal((M, D)).astype(np.float32)).to(torch.bfloat16))
    S = len(segs) - 1
    shift = nb(torch.from_numpy((0.1 * rng.standard_normal((S, D))).astype(np.float32)).to(torch.bfloat16))
    scale = nb(torch.from_numpy((0.1 * rng.standard_normal((S, D))).astype(np.float32)).to(torch.bfloat16))
    return x, np.array(segs, np.int64), shift, scale


def test_segment_selection_and_pack_match_torch_modulation(ora):
    x, rs, sh, sc = small_case(1)
    seg = ora.Segments(rs, sh, sc)
    y = torch_modulated(x, rs, sh, sc)
    amax = ora.modulate_amax(x, seg)
    assert amax == float(tb(y).float().abs().max())
    s_g = ora.tensor_scale(amax)
    q1, s1 = ora.modulate_pack_rows(x, seg, s_g, 0, 256)
    q2, s2 = ora.bf16_pack_rows(y, s_g, 0, 256)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_wrong_segment_boundary_changes_bytes(ora):
    """A boundary moved by one row changes the packed bytes of that row."""
    x, rs, sh, sc = small_case(2)
    seg = ora.Segments(rs, sh, sc)
    bad = ora.Segments(np.array([0, 38, 150, 200], np.int64), sh, sc)
    s_g = ora.tensor_scale(ora.modulate_amax(x, seg))
    q1, _ = ora.modulate_pack_rows(x, seg, s_g, 37, 38)
    q2, _ = ora.modulate_pack_rows(x, bad, s_g, 37, 38)
    assert not np.array_equal(q1, q2)


def test_nibble_order_and_row_major_layout(ora):
    """Blocks whose values are exactly E2M1 grid points (times one power of two
    through amax = 6) decode back to the same values: low nibble = even column,
    SFA row-major [rows, D/16], QDATA row-major [rows, D/2]."""
    vals = json.load(open(os.path.join(GOLD, "e2m1_values.json")))["values"]
    M, D = 3, 64
    grid = np.array([v * s for v in vals for s in (1, -1)], np.float32)
    rng = np.random.default_rng(4)
    yv = grid[rng.integers(0, grid.size, (M, D))]
    yv[:, ::16] = 6.0  # every block holds the global maximum
    y = nb(torch.from_numpy(yv).to(torch.bfloat16))
    s_g, q, s, amax = ora.quantize_bf16(y)
    assert amax == 6.0 and q.shape == (M, D // 2) and s.shape == (M, D // 16)
    assert np.all(s == 0x7E)
    e2 = np.array([ora.e2m1_value(c) for c in range(16)])
    dec = np.empty((M, D))
    dec[:, 0::2] = e2[q & 0xF]
    dec[:, 1::2] = e2[q >> 4]
    assert np.array_equal(dec, yv.astype(np.float64))


def test_padded_rows_zero_and_page_sizes(ora):
    sizes = json.load(open(os.path.join(GOLD, "page_sizes.json")))
    assert ora.padded_rows(sizes["canonical_rows"]) == sizes["padded_rows"]
    for k, mb in sizes["ring_slot_bytes_mb"].items():
        k = int(k)
        per_row = k // 2 + k // 16          # QDATA + SFA bytes per row
        assert per_row * 16 == 9 * k
        assert round(sizes["ring_rows"] * per_row / 1e6, 2) == mb
    full, last = divmod(sizes["canonical_rows"], sizes["ring_rows"])
    assert full + 1 == sizes["chunks"] and last == sizes["last_chunk_rows"]
    # the oracle's buffers have exactly those sizes and zero padding rows
    x, rs, sh, sc = small_case(3, M=70, D=32, segs=(0, 70))
    s_g, q, s, _ = ora.modulate_quantize(x, ora.Segments(rs, sh, sc))
    assert q.shape == (128, 16) and s.shape == (128, 2)
    assert not q[70:].any() and not s[70:].any()
    assert q[:70].any()


def test_global_scale_negative_control(ora):
    """Two-phase dependence: packing 32-row chunks with a per-chunk maximum
    instead of the global one changes the bytes of every chunk whose own
    maximum is below the global one."""
    x, rs, sh, sc = small_case(5, M=128, D=64, segs=(0, 128))
    x[7, 3] = nb(torch.tensor([300.0]).to(torch.bfloat16))[0]  # global max in chunk 0
    seg = ora.Segments(rs, sh, sc)
    s_g = ora.tensor_scale(ora.modulate_amax(x, seg))
    qg, sg_ = ora.modulate_pack_rows(x, seg, s_g, 0, 128)
    changed = 0
    for c0 in range(0, 128, 32):
        seg_c = ora.Segments(np.array([0, 32], np.int64), sh, sc)
        amax_c = ora.modulate_amax(x[c0:c0 + 32], seg_c)
        qc, scs = ora.modulate_pack_rows(x[c0:c0 + 32], seg_c, ora.tensor_scale(amax_c), 0, 32)
        same = np.array_equal(qc, qg[c0:c0 + 32]) and np.array_equal(scs, sg_[c0:c0 + 32])
        if c0 == 0:
            assert same
        else:
            assert not same
            changed += 1
    assert changed == 3


def test_zero_tensor(ora):
    M, D = 5, 32
    x = np.zeros((M, D), np.uint16)
    seg = ora.Segments(np.array([0, M], np.int64), np.zeros((1, D), np.uint16), np.zeros((1, D), np.uint16))
    s_g, q, s, amax = ora.modulate_quantize(x, seg)
    assert amax == 0.0 and s_g == 1.0
    assert not q.any() and not s.any()


def test_zero_block_with_shift_gives_shift(ora, syn):
    """x = 0 makes y = shift exactly; the tiny workload's zeroed block packs
    like the shift row it selects."""
    w = syn.workload("tiny")
    x = w.x()
    rs, sh, sc = w.segments()
    seg = ora.Segments(rs, sh, sc)
    s_g = ora.tensor_scale(ora.modulate_amax(x, seg))
    r, c0, c1 = w.zero_block
    assert not x[r, c0:c1].any()
    q, s = ora.modulate_pack_rows(x, seg, s_g, r, r + 1)
    yrow = x[r:r + 1].copy()
    yrow[0] = torch_modulated(x[r:r + 1], np.array([0, 1]), sh[0:1], sc[0:1])[0]
    assert np.array_equal(yrow[0, c0:c1], sh[0, c0:c1])
    q2, s2 = ora.bf16_pack_rows(yrow, s_g, 0, 1)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_swiglu_pack_matches_torch_swiglu_then_quantize(ora):
    rng = np.random.default_rng(6)
    M, F = 40, 64
    gu = nb(torch.from_numpy((2 * rng.standard_normal((M, 2 * F))).astype(np.float32)).to(torch.bfloat16))
    L = ora.lib()
    sb = np.array([L.ora_silu_bf16(int(g)) for g in gu[:, :F].ravel()], np.uint16).reshape(M, F)
    h = nb(tb(sb) * tb(gu[:, F:]))
    s_g, q, s, amax = ora.swiglu_quantize(gu)
    assert amax == float(tb(h).float().abs().max())
    s2, q2, ss2, _ = ora.quantize_bf16(h, m_pad=64)
    assert s_g == s2 and np.array_equal(q, q2) and np.array_equal(s, ss2)


# --------------------------------------------------------------------------
# GEMM reference
# --------------------------------------------------------------------------
def dequant_np(q, s, scale):
    """Dequantize with the published E2M1 table and torch's E4M3 decode."""
    vals = np.array(json.load(open(os.path.join(GOLD, "e2m1_values.json")))["values"])
    e2 = np.concatenate([vals, -vals])
    codes = np.empty((q.shape[0], q.shape[1] * 2), np.int64)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    sf = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return e2[codes] * np.repeat(sf, 16, axis=1), float(scale)


def _quantized_pair(ora, rng, M, N, K):
    a = nb(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16))
    w = nb(torch.from_numpy((0.02 * rng.standard_normal((N, K))).astype(np.float32)).to(torch.bfloat16))
    sa, qa, sfa, _ = ora.quantize_bf16(a)
    sw, qw, sfw, _ = ora.quantize_bf16(w)
    return sa, qa, sfa, sw, qw, sfw


def test_gemm_reference_matches_dequantized_matmul(ora):
    rng = np.random.default_rng(8)
    M, N, K = 24, 40, 96
    sa, qa, sfa, sw, qw, sfw = _quantized_pair(ora, rng, M, N, K)
    A, _ = dequant_np(qa, sfa, sa)
    W, _ = dequant_np(qw, sfw, sw)
    alpha = float(np.float32(sa) * np.float32(sw))
    want = alpha * (A @ W.T)
    rows = np.arange(M)
    got = ora.gemm_rows(qa, sfa, sa, qw, sfw, sw, rows)
    np.testing.assert_allclose(got, want, rtol=2 ** -40, atol=0)
    # a transposed weight or swapped rows would not match
    assert not np.allclose(ora.gemm_rows(qa, sfa, sa, qw, sfw, sw, rows[::-1]), want)


def test_gemm_identity_weight_returns_dequantized_activation(ora):
    """W = I: each weight row holds one 1.0, so s_w = RN(1/2688), its block gets
    sf = 448, the 1.0 encodes as 6 and decodes to 2688, and GEMM(A, I) equals
    the dequantized A up to the rounding of alpha (within tolerance)."""
    rng = np.random.default_rng(10)
    M, K = 16, 64
    a = nb(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16))
    sa, qa, sfa, _ = ora.quantize_bf16(a)
    eye = nb(torch.eye(K, dtype=torch.bfloat16))
    sw, qw, sfw, _ = ora.quantize_bf16(eye)
    assert sw == np.float32(1.0) / np.float32(2688.0)
    blocks = np.arange(K) // 16
    assert np.all(sfw[np.arange(K), blocks] == 0x7E)
    got = ora.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    A, _ = dequant_np(qa, sfa, sa)
    ok, worst = ora.gemm_tolerance_ok(got, A * float(sa))
    assert ok, worst
    np.testing.assert_allclose(got, A * float(sa), rtol=2 ** -22)


def test_gemm_bf16_output_for_an_identity_weight(ora):
    """With W = I each output is one product (plus K-1 exact zeros), exact in
    binary32, so the BF16 output is bf16(RN32(alpha * (2688 * A + 0))) with A
    the dequantized activation
    (torch's float32 -> bf16 cast as the rounding), and it lies within the
    half-ulp of the FP64 reference."""
    rng = np.random.default_rng(14)
    M, K = 20, 128
    a = nb(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32) * 3).to(torch.bfloat16))
    sa, qa, sfa, _ = ora.quantize_bf16(a)
    sw, qw, sfw, _ = ora.quantize_bf16(nb(torch.eye(K, dtype=torch.bfloat16)))
    got = ora.gemm_bf16_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    A, _ = dequant_np(qa, sfa, 1.0)
    alpha = np.float32(np.float32(sa) * np.float32(sw))
    # the sum over K adds +0 terms to the one product, so a -0 product sums to +0
    want = nb(torch.from_numpy((alpha * (A * 2688.0 + 0.0).astype(np.float32)).astype(np.float32)).to(torch.bfloat16))
    assert np.array_equal(got, want)
    ref = ora.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    gotf = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(gotf - ref) <= 2.0 ** -8 * np.abs(ref) * (1 + 2 ** -20))


def test_gate_residual_rows_selects_the_segment_gate(ora):
    """Row m uses the gate row of its segment; a shifted boundary changes rows."""
    rng = np.random.default_rng(15)
    M, N = 30, 48
    bf = lambda v: nb(torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16))  # noqa: E731
    o, res = bf(rng.standard_normal((M, N))), bf(rng.standard_normal((M, N)))
    gate = bf(rng.standard_normal((3, N)))
    rs = np.array([0, 7, 19, 30], np.int64)
    got = ora.gate_residual_rows(o, rs, gate, res)
    seg = np.searchsorted(rs[1:], np.arange(M), side="right")
    want = nb(tb(res) + tb(gate)[torch.from_numpy(seg)] * tb(o))
    assert np.array_equal(got, want)
    other = ora.gate_residual_rows(o, np.array([0, 8, 19, 30], np.int64), gate, res)
    assert not np.array_equal(other[7], got[7]) and np.array_equal(other[8:], got[8:])


def test_tolerance_rule_detects_a_dropped_block(ora):
    """The GEMM tolerance rejects an output that misses one 16-wide K block."""
    rng = np.random.default_rng(12)
    M, N, K = 8, 32, 128
    sa, qa, sfa, sw, qw, sfw = _quantized_pair(ora, rng, M, N, K)
    ref = ora.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    qa2 = qa.copy()
    qa2[:, 8:16] = 0  # drop block 1
    bad = ora.gemm_rows(qa2, sfa, sa, qw, sfw, sw, np.arange(M))
    assert ora.gemm_tolerance_ok(ref, ref)[0]
    assert not ora.gemm_tolerance_ok(bad, ref)[0]


@pytest.mark.parametrize("name", ["tiny"])
def test_tiny_workload_end_to_end_oracle(ora, syn, name):
    """The tiny workload runs through the whole oracle: the outliers dominate
    the tensor scale and the output has the expected shape."""
    w = syn.workload(name)
    x = w.x()
    rs, sh, sc = w.segments()
    s_g, q, s, amax = ora.modulate_quantize(x, ora.Segments(rs, sh, sc))
    assert 50.0 <= amax <= 400.0
    assert q.shape == (256, 256) and s.shape == (256, 32)
    sw, qw, sfw, _ = ora.quantize_bf16(w.weight())
    out = ora.gemm_rows(q, s, s_g, qw, sfw, sw, np.arange(0, 256, 17))
    assert out.shape == (16, 1024) and np.isfinite(out).all()
