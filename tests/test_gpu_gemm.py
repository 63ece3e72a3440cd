"""The block-scaled GEMM against the FP64 oracle:
|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), ref = RN32(s_a*s_w) * sum_k A*W in
binary64 (not rounded to bf16), rms over the checked outputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _par
from tests.gpu_util import device, first_mismatch, host, host_u16, to_dev, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import nvfp4_activation_quantization_segment_amd as pkg

    device()
    return pkg


def bf16_np(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def out_f64(t):
    return (host_u16(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check(ref, got, what=""):
    ok, worst = oracle.gemm_tolerance_ok(got, ref)
    assert ok, f"{what}: worst |err|/bound = {worst:.3g}"
    return worst


def oracle_quantized(a, w, m_pad):
    sa, qa, sfa, _ = _par.quantize_bf16(a, m_pad)
    sw, qw, sfw, _ = _par.quantize_bf16(w)
    return sa, qa, sfa, sw, qw, sfw


def gpu_gemm(m, sa, qa, sfa, sw, qw, sfw, M, ldo=None):
    dev = device()
    N = qw.shape[0]
    ldo = N if ldo is None else ldo
    out = torch.full((M, ldo), float("nan"), dtype=torch.bfloat16, device=dev)
    m.nvfp4_gemm(to_dev(qa), to_dev(sfa), to_dev(np.array([sa], np.float32)), M, qa.shape[0], to_dev(qw),
                 to_dev(sfw), to_dev(np.array([sw], np.float32)), N, 2 * qw.shape[1], out, ldo)
    torch.cuda.synchronize()
    return out


def test_tiny_workload_end_to_end_all_outputs(m):
    """Tiny workload: GPU producer -> GPU GEMM, all 256 x 1024 outputs."""
    w = synth.workload("tiny")
    x = w.x()
    rs, sh, sc = w.segments()
    W = w.weight()
    q, s, ts, _ = m.modulate_quantize(to_dev_u16(x), rs, to_dev_u16(sh), to_dev_u16(sc))
    qw, sfw, tw = m.quantize_weight(to_dev_u16(W))
    out = m.gemm(q, s, ts, w.M, qw, sfw, tw)
    torch.cuda.synchronize()
    s_g, oq, osf, _ = oracle.modulate_quantize(x, oracle.Segments(rs, sh, sc))
    sw, oqw, osfw, _ = oracle.quantize_bf16(W)
    ref = _par.gemm_rows(oq, osf, s_g, oqw, osfw, sw, np.arange(w.M))
    check(ref, out_f64(out), "tiny")


@pytest.mark.parametrize("M,N,K", [
    (1, 16, 64), (37, 48, 192), (300, 272, 128), (257, 1024, 512), (64, 16, 5376), (130, 528, 14336),
])
def test_ragged_shapes(m, M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    m_pad = oracle.padded_rows(M)
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, m_pad)
    out = gpu_gemm(m, sa, qa, sfa, sw, qw, sfw, M)
    ref = _par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    check(ref, out_f64(out), f"{M}x{N}x{K}")


@pytest.mark.parametrize("extra", [8, 4])
def test_output_stride_and_untouched_padding(m, extra):
    """ldo > N: the columns beyond N are not written.  ldo = N + 8 takes the
    epilogue that writes whole 16-byte chunks; ldo = N + 4 (rows only 8-byte
    aligned) the one that writes 8 bytes per lane."""
    rng = np.random.default_rng(5)
    M, N, K = 70, 64, 128
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, 128)
    out = gpu_gemm(m, sa, qa, sfa, sw, qw, sfw, M, ldo=N + extra)
    got = out_f64(out)
    assert np.isnan(got[:, N:]).all()
    check(_par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M)), got[:, :N])


def test_output_base_8_byte_aligned(m):
    """An output base that is 8- but not 16-byte aligned takes the 8-byte
    epilogue; the results match, and nothing before the base is written."""
    rng = np.random.default_rng(15)
    M, N, K = 300, 272, 128
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))
    dev = device()
    buf = torch.full((M * N + 8,), float("nan"), dtype=torch.bfloat16, device=dev)
    out = buf[4:4 + M * N].view(M, N)
    assert out.data_ptr() % 16 == 8
    m.nvfp4_gemm(to_dev(qa), to_dev(sfa), to_dev(np.array([sa], np.float32)), M, qa.shape[0], to_dev(qw),
                 to_dev(sfw), to_dev(np.array([sw], np.float32)), N, K, out, N)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:4]).all() and torch.isnan(buf[4 + M * N:]).all()
    check(_par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M)), out_f64(out))


def test_identity_weight_returns_dequantized_activation(m):
    rng = np.random.default_rng(6)
    M, K = 96, 256
    a = bf16_np(rng.standard_normal((M, K)))
    eye = bf16_np(np.eye(K))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, eye, 128)
    out = gpu_gemm(m, sa, qa, sfa, sw, qw, sfw, M)
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)])
    codes = np.empty((M, K), np.int64)
    codes[:, 0::2] = qa[:M] & 0xF
    codes[:, 1::2] = qa[:M] >> 4
    sf = np.array([oracle.e4m3_value(c) for c in range(256)])[sfa[:M]]
    deq = e2[codes] * np.repeat(sf, 16, axis=1) * float(sa)
    check(deq, out_f64(out), "identity")


def test_zero_activation_gives_zero(m):
    M, N, K = 64, 32, 64
    qa = np.zeros((M, K // 2), np.uint8)
    sfa = np.zeros((M, K // 16), np.uint8)
    rng = np.random.default_rng(7)
    w = bf16_np(rng.standard_normal((N, K)))
    sw, qw, sfw, _ = _par.quantize_bf16(w)
    out = gpu_gemm(m, 1.0, qa, sfa, sw, qw, sfw, M)
    assert (out_f64(out) == 0).all()


def test_signed_and_nan_scale_bytes_decode_as_the_oracle(m):
    """Scale bytes the producer never writes, read as E4M3FN like the oracle
    reads them: the sign bit gives a negative scale and 0x7F (the NaN code)
    makes every product with its block NaN, so one NaN activation scale turns
    its output row into NaN and one NaN weight scale its output column."""
    rng = np.random.default_rng(31)
    M, N, K = 96, 48, 256
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.05 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))
    sfa, sfw = sfa.copy(), sfw.copy()
    sfa[rng.random(sfa.shape) < 0.3] |= 0x80
    sfw[rng.random(sfw.shape) < 0.3] |= 0x80
    sfa[5, 3] = 0x7F
    sfw[7, 0] = 0x7F
    ref = _par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    nan = np.isnan(ref)
    assert nan[5].all() and nan[:, 7].all() and nan.sum() == M + N - 1
    ref_u = _par.gemm_rows(qa, sfa & 0x7F, sa, qw, sfw & 0x7F, sw, np.arange(M))
    assert not np.allclose(ref[~nan], ref_u[~nan])  # the sign bits change the sums
    out = out_f64(gpu_gemm(m, sa, qa, sfa, sw, qw, sfw, M))
    assert np.array_equal(np.isnan(out), nan)
    check(ref[~nan], out[~nan], "signed scale bytes")


def test_extreme_scales_fp16_range(m):
    """Largest and smallest decoded magnitudes (6*448 and 0.5*2^-9) on both
    operands stay exact through the fp16 decode."""
    M, N, K = 64, 16, 64
    qa = np.full((M, K // 2), 0x77, np.uint8)     # +6, +6
    sfa = np.full((M, K // 16), 0x7E, np.uint8)   # 448
    qw = np.full((N, K // 2), 0x11, np.uint8)     # +0.5
    sfw = np.full((N, K // 16), 0x01, np.uint8)   # 2^-9
    out = gpu_gemm(m, 1.0, qa, sfa, 1.0, qw, sfw, M)
    ref = _par.gemm_rows(qa, sfa, 1.0, qw, sfw, 1.0, np.arange(M))
    assert np.allclose(ref, 2688.0 * 2.0 ** -10 * K)
    check(ref, out_f64(out), "extremes")


@pytest.mark.parametrize("name", ["qkv", "fc1", "fc2"])
def test_canonical_projection_sampled_rows(m, name):
    """Producer + GEMM at M = 37,810 on one stream; 64 checked rows (boundary
    rows 0, 1, 63, 64, 30999, 31000, 37807-37809 plus seeded rows), all N."""
    w = synth.workload(name)
    dev = device()
    print(f"{name}: M={w.M} K={w.K} N={w.N}", flush=True)
    if w.kind == "modulate":
        x = w.x()
        rs, sh, sc = w.segments()
        q, s, ts, _ = m.modulate_quantize(to_dev_u16(x), rs, to_dev_u16(sh), to_dev_u16(sc))
    else:
        gu = w.gate_up()
        q, s, ts, _ = m.swiglu_quantize(to_dev_u16(gu))
    W = w.weight()
    qw, sfw, tw = m.quantize_weight(to_dev_u16(W))
    out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    m.gemm(q, s, ts, w.M, qw, sfw, tw, out=out)
    torch.cuda.synchronize()
    rows = w.check_rows(64)
    # oracle side: its own tensor scale over every row, its own bytes for the
    # checked rows, its own weight quantization
    if w.kind == "modulate":
        seg = oracle.Segments(rs, sh, sc)
        amax = _par.amax_merge(_par._map(lambda r: oracle.modulate_amax_rows(x, seg, *r), _par._ranges(w.M, 64)))
        sa = oracle.tensor_scale(amax)
        parts = _par._map(lambda r: oracle.modulate_pack_rows(x, seg, sa, r, r + 1), list(rows))
    else:
        amax = _par.amax_merge(_par._map(lambda r: oracle.swiglu_amax_rows(gu, *r), _par._ranges(w.M, 64)))
        sa = oracle.tensor_scale(amax)
        parts = _par._map(lambda r: oracle.swiglu_pack_rows(gu, sa, r, r + 1), list(rows))
    assert np.float32(sa) == host(ts)[0]
    oqa = np.concatenate([p[0] for p in parts])
    osfa = np.concatenate([p[1] for p in parts])
    sw, oqw, osfw, _ = _par.quantize_bf16(W)
    assert sw == host(tw)[0]
    assert np.array_equal(oqw, host(qw)) and np.array_equal(osfw, host(sfw))
    ref = _par.gemm_rows(oqa, osfa, sa, oqw, osfw, sw, np.arange(rows.size))
    got = out_f64(out[torch.from_numpy(rows).to(dev)])
    worst = check(ref, got, name)
    print(f"{name}: worst err/bound {worst:.3g}", flush=True)


def _decoded(q, sf, rows, K, e2m1):
    """Exact binary32 values of packed rows: E2M1 codes (low nibble first)
    through the published value set, times the E4M3 scale of each 16."""
    codes = torch.stack([(q[:rows] & 0xF).long(), (q[:rows] >> 4).long()], dim=-1).reshape(rows, K)
    scale = sf[:rows].view(torch.float8_e4m3fn).to(torch.float32).repeat_interleave(16, dim=1)
    return e2m1[codes] * scale


@pytest.mark.parametrize("name", ["qkv", "fc1", "fc2"])
def test_canonical_projection_every_output_against_fp32_product(m, name):
    """Every output of the projection at M = 37,810 (the launches bench.py
    times: main, K-split tail and finalize) against a binary32 product of the
    exactly decoded operands, under the same tolerance with the rms taken over
    all outputs.  The product is torch's fp32 matmul on the GPU (TF32 off); the
    decode uses the published E2M1 values and torch's float8 decode, and each
    decoded value is exact in binary32.  The oracle comparison samples rows;
    this reaches every tile, the ragged last row tile and the split tail tiles
    included.  The packed operands are the producer's and the weight
    quantizer's, whose bytes the producer tests compare with the oracle."""
    import json
    import os

    w = synth.workload(name)
    dev = device()
    print(f"{name}: every output, M={w.M} K={w.K} N={w.N}", flush=True)
    if w.kind == "modulate":
        rs, sh, sc = w.segments()
        q, s, ts, _ = m.modulate_quantize(to_dev_u16(w.x()), rs, to_dev_u16(sh), to_dev_u16(sc))
    else:
        q, s, ts, _ = m.swiglu_quantize(to_dev_u16(w.gate_up()))
    qw, sfw, tw = m.quantize_weight(to_dev_u16(w.weight()))
    out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    m.gemm(q, s, ts, w.M, qw, sfw, tw, out=out)
    torch.cuda.synchronize()
    with open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.json")) as f:
        mags = json.load(f)["values"]
    e2m1 = torch.tensor(mags + [-v for v in mags], dtype=torch.float32, device=dev)
    alpha = torch.tensor(np.float32(host(ts)[0]) * np.float32(host(tw)[0]), dtype=torch.float32, device=dev)
    wdec = _decoded(qw, sfw, w.N, w.K, e2m1)
    tf32 = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        excess, sumsq = -np.inf, 0.0
        for r0 in range(0, w.M, 4096):
            r1 = min(w.M, r0 + 4096)
            ref = (_decoded(q[r0:], s[r0:], r1 - r0, w.K, e2m1) @ wdec.t()) * alpha
            got = out[r0:r1].float()
            excess = max(excess, float(((got - ref).abs() - 2.0 ** -7 * ref.abs()).max()))
            sumsq += float((ref.double() ** 2).sum())
    finally:
        torch.backends.cuda.matmul.allow_tf32 = tf32
    rms = (sumsq / (w.M * w.N)) ** 0.5
    print(f"{name}: worst excess over 2^-7|ref| {excess:.3g}, 1e-3 rms {1e-3 * rms:.3g}", flush=True)
    assert excess <= 1e-3 * rms, (excess, rms)


def test_scale_rows_misaligned_take_the_word_path(m):
    """K % 256 == 0 lets the kernel fetch scales 16 bytes per row per 4 K
    steps, but only when both scale arrays are 16-byte aligned; scale arrays
    that are only 4-byte aligned take the 4-byte path.  Both give the same
    bits (the accumulation order does not depend on how scales are loaded)."""
    dev = device()
    rng = np.random.default_rng(11)
    M, N, K = 200, 272, 512
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))

    def offset_copy(arr, off):
        buf = torch.zeros(arr.size + 64, dtype=torch.uint8, device=dev)
        view = buf[off:off + arr.size].view(arr.shape)
        view.copy_(torch.from_numpy(np.ascontiguousarray(arr)))
        assert view.data_ptr() % 16 == off % 16
        return view

    outs = []
    for off in (0, 4):
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        m.nvfp4_gemm(to_dev(qa), offset_copy(sfa, off), to_dev(np.array([sa], np.float32)), M, qa.shape[0],
                     to_dev(qw), offset_copy(sfw, off), to_dev(np.array([sw], np.float32)), N, K, out, N)
        torch.cuda.synchronize()
        outs.append(host_u16(out))
    ref = _par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    for o in outs:
        check(ref, (o.astype(np.uint32) << 16).view(np.float32).astype(np.float64), "alignment")
    assert np.array_equal(outs[0], outs[1])


def gpu_gemm_ws(m, sa, qa, sfa, sw, qw, sfw, M, workspace_pad=0):
    dev = device()
    N = qw.shape[0]
    K = 2 * qw.shape[1]
    need = m.nvfp4_gemm_workspace_bytes(M, N, K)
    ws = torch.full((need + workspace_pad,), 0xFF, dtype=torch.uint8, device=dev) if need else None
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    m.nvfp4_gemm_ws(to_dev(qa), to_dev(sfa), to_dev(np.array([sa], np.float32)), M, qa.shape[0], to_dev(qw),
                    to_dev(sfw), to_dev(np.array([sw], np.float32)), N, K, out, N, ws, need)
    torch.cuda.synchronize()
    return out, need


@pytest.mark.parametrize("M,N,K", [
    (64, 16, 5376), (130, 528, 14336), (257, 1024, 512), (600, 4096, 1024), (300, 272, 128), (1, 16, 64),
    (200, 512, 640),  # K/16 = 40: 4-byte scale path inside the K-split pieces (pieces of 8 and 2 steps)
])
def test_split_tail_small_shapes(m, M, N, K):
    """nvfp4_gemm_ws on shapes whose single partial wave is split along K
    (and two that are not split), every output against the FP64 oracle."""
    rng = np.random.default_rng(3 * M + N + K)
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))
    out, need = gpu_gemm_ws(m, sa, qa, sfa, sw, qw, sfw, M)
    print(f"{M}x{N}x{K}: workspace {need} bytes", flush=True)
    check(_par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M)), out_f64(out), f"ws {M}x{N}x{K}")


def test_split_tail_after_full_waves(m):
    """272 tiles = one full wave of 256 and 16 tail tiles (the last M-tile row),
    each split into 4 K ranges.  Tiles of the full wave are bit-identical to
    nvfp4_gemm; the tail rows match the oracle."""
    rng = np.random.default_rng(17)
    M, N, K = 17 * 256, 16 * 256, 1024
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))
    out_ws, need = gpu_gemm_ws(m, sa, qa, sfa, sw, qw, sfw, M, workspace_pad=4096)
    assert need == 16 * 4 * 8 * 128 * 64 * 4
    out_plain = gpu_gemm(m, sa, qa, sfa, sw, qw, sfw, M)
    got_ws, got_plain = host_u16(out_ws), host_u16(out_plain)
    assert np.array_equal(got_ws[:16 * 256], got_plain[:16 * 256])
    rows = np.concatenate([np.arange(16 * 256, M, 3), np.array([0, 1, 255, 4095])])
    ref = _par.gemm_rows(qa, sfa, sa, qw, sfw, sw, rows)
    check(ref, (got_ws[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64), "tail rows")
    check(ref, (got_plain[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64), "plain rows")


def test_convenience_gemm_on_a_non_current_stream(m):
    """gemm(stream=s) with s not the current stream: the K-split workspace it
    allocates belongs to s, so allocations and writes on the current stream
    while s still runs (here behind a long matrix product) cannot take it over.
    The output is bit-identical to the same call on the current stream."""
    dev = device()
    rng = np.random.default_rng(29)
    M, N, K = 2560, 6656, 1024
    need = m.nvfp4_gemm_workspace_bytes(M, N, K)
    assert need > 0
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))
    args = (to_dev(qa), to_dev(sfa), to_dev(np.array([sa], np.float32)), M, to_dev(qw), to_dev(sfw),
            to_dev(np.array([sw], np.float32)))
    want = host_u16(m.gemm(*args))
    side = torch.cuda.Stream(device=dev)
    big = torch.randn((6144, 6144), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        busy = big @ big                      # keeps the side stream busy for a while
    out = m.gemm(*args, stream=side)
    for i in range(200):                      # reuse pressure on the current stream meanwhile
        t = torch.empty(need, dtype=torch.uint8, device=dev)
        t.fill_(0x7F)
        torch.cuda._sleep(20000)
        del t
    torch.cuda.synchronize()
    del busy
    got = host_u16(out)
    assert np.array_equal(got, want), first_mismatch(got, want)


def test_split_tail_with_4byte_aligned_scales(m):
    """The K-split pieces with scale arrays that are only 4-byte aligned (the
    per-step scale path, offset to each piece's first K step)."""
    dev = device()
    rng = np.random.default_rng(23)
    M, N, K = 300, 768, 2048
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))
    need = m.nvfp4_gemm_workspace_bytes(M, N, K)
    assert need > 0

    def offset_copy(arr, off):
        buf = torch.zeros(arr.size + 64, dtype=torch.uint8, device=dev)
        view = buf[off:off + arr.size].view(arr.shape)
        view.copy_(torch.from_numpy(np.ascontiguousarray(arr)))
        return view

    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    m.nvfp4_gemm_ws(to_dev(qa), offset_copy(sfa, 4), to_dev(np.array([sa], np.float32)), M, qa.shape[0], to_dev(qw),
                    offset_copy(sfw, 4), to_dev(np.array([sw], np.float32)), N, K, out, N, ws, need)
    torch.cuda.synchronize()
    check(_par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M)), out_f64(out), "ws misaligned scales")


# --------------------------------------------------------------------------
# Exact residual epilogue: out = bf16(residual + bf16(gate[s][n] * o))
# --------------------------------------------------------------------------
def gpu_gate_residual(m, sa, qa, sfa, sw, qw, sfw, M, rs, gate, residual, ldo=None, in_place=False):
    dev = device()
    N, K = qw.shape[0], 2 * qw.shape[1]
    ldo = N if ldo is None else ldo
    res = torch.full((M, ldo), float("nan"), dtype=torch.bfloat16, device=dev)
    res[:, :N] = to_dev_u16(residual)
    out = res if in_place else torch.full((M, ldo), float("nan"), dtype=torch.bfloat16, device=dev)
    gates, keep = m.make_row_gates(rs, to_dev_u16(gate))
    need = m.nvfp4_gemm_workspace_bytes(M, N, K)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    m.nvfp4_gemm_gate_residual(to_dev(qa), to_dev(sfa), to_dev(np.array([sa], np.float32)), M, qa.shape[0],
                               to_dev(qw), to_dev(sfw), to_dev(np.array([sw], np.float32)), N, K, gates, res, ldo,
                               out, ldo, ws, need)
    torch.cuda.synchronize()
    del keep
    return host_u16(out)


@pytest.mark.parametrize("M,K,segs,extra,in_place", [
    (200, 256, (0, 37, 150, 200), 0, False),     # 16-byte staged stores
    (200, 256, (0, 37, 150, 200), 0, True),      # out is the residual
    (130, 192, (0, 1, 129, 130), 4, False),      # rows 8-byte aligned only: 8-byte stores
    (64, 5376, (0, 20, 64), 0, False),           # one row of tiles: K-split pieces and the finalize kernel
])
def test_gate_residual_identity_weight_bit_exact(m, M, K, segs, extra, in_place):
    """With W = I every output is one product, so the GEMM's bf16 output is
    exact and the fused epilogue is compared with the oracle bit for bit."""
    rng = np.random.default_rng(M + K)
    a = bf16_np(3 * rng.standard_normal((M, K)))
    sa, qa, sfa, _ = _par.quantize_bf16(a, oracle.padded_rows(M))
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    sw, qw, sfw, _ = _par.quantize_bf16(eye)
    S = len(segs) - 1
    gate = bf16_np(1 + 0.3 * rng.standard_normal((S, K)))
    residual = bf16_np(rng.standard_normal((M, K)))
    rs = np.array(segs, np.int64)
    o = _par.gemm_bf16_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    want = oracle.gate_residual_rows(o, rs, gate, residual)
    got = gpu_gate_residual(m, sa, qa, sfa, sw, qw, sfw, M, rs, gate, residual, ldo=K + extra, in_place=in_place)
    assert np.array_equal(got[:, :K], want), first_mismatch(got[:, :K], want)
    if extra:
        assert np.isnan((got[:, K:].astype(np.uint32) << 16).view(np.float32)).all()


def test_gate_residual_random_within_tolerance(m):
    """Random operands: out against the FP64 reference residual + gate * ref,
    within the GEMM tolerance carried through the gate product plus one bf16
    half-ulp for each of the two further roundings."""
    rng = np.random.default_rng(31)
    M, N, K = 300, 272, 512
    a = bf16_np(rng.standard_normal((M, K)))
    w = bf16_np(0.02 * rng.standard_normal((N, K)))
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, oracle.padded_rows(M))
    rs = np.array([0, 100, 300], np.int64)
    gate = bf16_np(0.5 * rng.standard_normal((2, N)))
    residual = bf16_np(rng.standard_normal((M, N)))
    got = (gpu_gate_residual(m, sa, qa, sfa, sw, qw, sfw, M, rs, gate, residual).astype(np.uint32) << 16)
    got = got.view(np.float32).astype(np.float64)
    ref_o = _par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    seg = np.searchsorted(rs[1:], np.arange(M), side="right")
    g = (gate.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[seg]
    r = (residual.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = r + g * ref_o
    e_o = 2.0 ** -7 * np.abs(ref_o) + 1e-3 * np.sqrt(np.mean(ref_o ** 2))
    e_g = np.abs(g) * e_o + 2.0 ** -8 * np.abs(g) * (np.abs(ref_o) + e_o)
    bound = e_g + 2.0 ** -8 * (np.abs(ref) + e_g) + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= bound), float(np.max(err / bound))


def test_attention_output_projection_with_residual_epilogue(m):
    """The attention-output projection at M = 37,810, K = 7,168, N = 5,376: the
    plain quantizer, then the GEMM with the residual epilogue (two segments of
    gates).  The packed activation is compared byte for byte with the oracle's
    on the checked rows, the outputs against the FP64 reference
    residual + gate * ref within the tolerance of the epilogue test above."""
    w = synth.workload("attn_out")
    dev = device()
    x = w.x()
    W = w.weight()
    rs, gate = w.gates()
    residual = w.residual()
    print(f"attn_out: M={w.M} K={w.K} N={w.N}", flush=True)
    q, s, ts, _ = m.quantize(to_dev_u16(x))
    qw, sfw, tw = m.quantize_weight(to_dev_u16(W))
    res = to_dev_u16(residual)
    gates, keep = m.make_row_gates(rs, to_dev_u16(gate))
    need = m.nvfp4_gemm_workspace_bytes(w.M, w.N, w.K)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    m.nvfp4_gemm_gate_residual(q, s, ts, w.M, q.shape[0], qw, sfw, tw, w.N, w.K, gates, res, w.N, res, w.N, ws,
                               need)
    torch.cuda.synchronize()
    rows = w.check_rows(64)
    sa, oqa, osfa, _ = _par.quantize_bf16(x, w.m_pad)
    assert np.float32(sa) == host(ts)[0]
    assert np.array_equal(host(q)[rows], oqa[rows]) and np.array_equal(host(s)[rows], osfa[rows])
    sw, oqw, osfw, _ = _par.quantize_bf16(W)
    assert sw == host(tw)[0]
    ref_o = _par.gemm_rows(oqa, osfa, sa, oqw, osfw, sw, rows)
    seg = np.searchsorted(rs[1:], rows, side="right")
    g = (gate.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[seg]
    r = (residual[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = r + g * ref_o
    got = out_f64(res[torch.from_numpy(rows).to(dev)])
    e_o = 2.0 ** -7 * np.abs(ref_o) + 1e-3 * np.sqrt(np.mean(ref_o ** 2))
    e_g = np.abs(g) * e_o + 2.0 ** -8 * np.abs(g) * (np.abs(ref_o) + e_o)
    bound = e_g + 2.0 ** -8 * (np.abs(ref) + e_g) + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
    del keep


def test_activation_past_4_gib_runs_in_row_chunks(m):
    """M = 600,000 rows at K = 14,336: the packed activation (4.30 GB) exceeds
    the kernel's 32-bit offsets and runs as two row chunks (599,040 + 960
    rows).  A repeats a seeded 61-row block (tiled on the device; the oracle
    runs on the block).  nvfp4_gemm_ws with random weights against the FP64
    oracle on rows sampled on both sides of the chunk boundary; the residual
    epilogue with a partial identity weight (every output one product, so
    bit-exact) and a gate segment boundary inside the second chunk."""
    dev = device()
    M, N, K, P = 600_000, 256, 14336, 61
    m_pad = oracle.padded_rows(M)
    assert m_pad * K // 2 > 1 << 32
    a = synth.add_outliers_t3(synth.normal_bf16(50, 0, (P, K), 1.0), 50, 0.001, 20.0)
    sa, qa, sfa, _ = _par.quantize_bf16(a, P)
    reps = -(-m_pad // P)
    qa_d = to_dev(qa).repeat(reps, 1)[:m_pad].contiguous()
    sfa_d = to_dev(sfa).repeat(reps, 1)[:m_pad].contiguous()
    sa_d = to_dev(np.array([sa], np.float32))
    rows = np.unique(np.concatenate([
        np.array([0, 1, 255, 256, 599_039, 599_040, 599_041, 599_099, 599_100, M - 2, M - 1]),
        synth.sample_rows(51, M, 96)]))
    ridx = torch.from_numpy(rows).to(dev)
    print(f"A [{m_pad}, {K // 2}] packed, {rows.size} checked rows", flush=True)

    w = bf16_np(0.02 * np.random.default_rng(52).standard_normal((N, K)))
    sw, qw, sfw, _ = _par.quantize_bf16(w)
    need = m.nvfp4_gemm_workspace_bytes(M, N, K)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    m.nvfp4_gemm_ws(qa_d, sfa_d, sa_d, M, m_pad, to_dev(qw), to_dev(sfw), to_dev(np.array([sw], np.float32)), N, K,
                    out, N, ws, need)
    torch.cuda.synchronize()
    check(_par.gemm_rows(qa, sfa, sa, qw, sfw, sw, rows % P), out_f64(out[ridx]), "row chunks")
    del out

    eye = np.zeros((N, K), np.uint16)
    eye[np.arange(N), np.arange(N)] = 0x3F80
    sw, qw, sfw, _ = _par.quantize_bf16(eye)
    rs = np.array([0, 599_100, M], np.int64)
    gate = bf16_np(1 + 0.3 * np.random.default_rng(53).standard_normal((2, N)))
    rblock = synth.normal_bf16(54, 0, (P, N), 1.0)
    res = to_dev_u16(rblock).repeat(reps, 1)[:M].contiguous()
    gates, keep = m.make_row_gates(rs, to_dev_u16(gate))
    m.nvfp4_gemm_gate_residual(qa_d, sfa_d, sa_d, M, m_pad, to_dev(qw), to_dev(sfw),
                               to_dev(np.array([sw], np.float32)), N, K, gates, res, N, res, N, ws, need)
    torch.cuda.synchronize()
    del keep
    o = _par.gemm_bf16_rows(qa, sfa, sa, qw, sfw, sw, rows % P)
    seg_rs = np.array([0, int(np.searchsorted(rows, 599_100)), rows.size], np.int64)
    want = oracle.gate_residual_rows(o, seg_rs, gate, rblock[rows % P])
    got = host_u16(res[ridx])
    assert np.array_equal(got, want), first_mismatch(got, want)


def test_gemm_ws_under_graph_capture_replays_match_eager(m):
    """nvfp4_gemm_ws captured into a HIP graph on a shape whose last wave of
    tiles is split along K (256 whole tiles and 4 split ones, then the
    finalize launch): four replays with new operands copied into the captured
    buffers, each bit for bit equal to the same call run eagerly in between.
    The library enqueues kernels only (no memset), so the graph holds kernels
    only."""
    dev = device()
    M, N, K = 13 * 256, 20 * 256, 1024
    m_pad = oracle.padded_rows(M)
    nbytes = int(m.nvfp4_gemm_workspace_bytes(M, N, K))
    assert nbytes > 0
    bufs = {}

    def load(seed):
        rng = np.random.default_rng(seed)
        a = bf16_np(rng.standard_normal((M, K)))
        w = bf16_np(0.05 * rng.standard_normal((N, K)))
        sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, m_pad)
        vals = dict(qa=qa, sfa=sfa, qw=qw, sfw=sfw, sa=np.array([sa], np.float32), sw=np.array([sw], np.float32))
        for k, v in vals.items():
            t = torch.from_numpy(np.ascontiguousarray(v))
            if k in bufs:
                bufs[k].copy_(t)
            else:
                bufs[k] = t.to(dev)

    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_eager = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def call(o, wsp):
        b = bufs
        m.nvfp4_gemm_ws(b["qa"], b["sfa"], b["sa"], M, m_pad, b["qw"], b["sfw"], b["sw"], N, K, o, N, wsp, nbytes)

    load(200)
    call(out, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # captured on the graph's own stream, the current one inside
        call(out, ws)
    torch.cuda.synchronize()
    for rep, seed in enumerate((201, 202, 203, 204)):
        print(f"replay {rep} with operand seed {seed}", flush=True)
        load(seed)
        torch.cuda.synchronize()
        call(ref, ws_eager)  # eager work between the replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
