"""The packed-tile ring (nvfp4_modulate_gemm_ring) against the oracle and the
materialized path: every chunk's slot bytes against the oracle's QDATA/SFA
rows, the outputs against the chained producer + GEMM (bit for bit where
neither splits tiles along K) and against the FP64 oracle within the GEMM
tolerance, and the same outputs whatever the number of slots."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _par
from tests.gpu_util import device, first_mismatch, host, host_u16, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import nvfp4_activation_quantization_segment_amd as pkg

    device()
    return pkg


def out_f64(t):
    return (host_u16(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def slot_views(ring, slots, chunk_rows, K):
    """(qdata [chunk_rows, K/2], sfa [chunk_rows, K/16]) views of each slot."""
    sb = chunk_rows * (K // 2 + K // 16)
    views = []
    for i in range(slots):
        b = ring[i * sb:(i + 1) * sb]
        views.append((b[:chunk_rows * (K // 2)].view(chunk_rows, K // 2),
                      b[chunk_rows * (K // 2):].view(chunk_rows, K // 16)))
    return views


def check_slots(ring, chunk_rows, M, K, oq, osf):
    """With at least as many slots as chunks, slot c holds chunk c's rows of
    the oracle's QDATA/SFA, then zero rows up to the next multiple of 64."""
    chunks = -(-M // chunk_rows)
    views = slot_views(ring, chunks, chunk_rows, K)
    for c in range(chunks):
        r0 = c * chunk_rows
        rows = min(M, r0 + chunk_rows) - r0
        pad = -(-rows // 64) * 64
        q, s = host(views[c][0][:pad]), host(views[c][1][:pad])
        assert np.array_equal(s[:rows], osf[r0:r0 + rows]), (c, "SFA", first_mismatch(s[:rows], osf[r0:r0 + rows]))
        assert np.array_equal(q[:rows], oq[r0:r0 + rows]), (c, "QDATA", first_mismatch(q[:rows], oq[r0:r0 + rows]))
        assert not q[rows:].any() and not s[rows:].any(), (c, "padding rows")


def test_ring_small_ragged_chunks_and_segments(m):
    """M = 1000 in chunks of 256 (the last of 232 rows), three segments whose
    bounds fall inside chunks; slots = chunks, then 2 and 1."""
    dev = device()
    M, K, N, chunk = 1000, 256, 512, 256
    x = synth.add_outliers_t3(synth.normal_bf16(71, 0, (M, K), 1.0), 71, 0.01, 20.0)
    sh = synth.normal_bf16(71, 1, (3, K), 0.1)
    sc = synth.normal_bf16(71, 2, (3, K), 0.1)
    W = synth.normal_bf16(71, 3, (N, K), 0.02)
    rs = [0, 300, 700, M]
    xd, shd, scd = to_dev_u16(x), to_dev_u16(sh), to_dev_u16(sc)
    qw, sfw, tw = m.quantize_weight(to_dev_u16(W))
    # oracle bytes
    seg = oracle.Segments(rs, sh, sc)
    s_g, oq, osf, _ = _par.modulate_quantize(x, seg, oracle.padded_rows(M))
    chunks = -(-M // chunk)
    out_full, ts, amax, ring = m.modulate_gemm_ring(xd, rs, shd, scd, qw, sfw, tw, chunk_rows=chunk, slots=chunks)
    torch.cuda.synchronize()
    assert host(ts)[0] == np.float32(s_g)
    check_slots(ring, chunk, M, K, oq, osf)
    # the chained path: producer, then one GEMM over all rows
    q, s, ts2, _ = m.modulate_quantize(xd, rs, shd, scd)
    chained = m.gemm(q, s, ts2, M, qw, sfw, tw)
    torch.cuda.synchronize()
    assert torch.equal(out_full.view(torch.int16), chained.view(torch.int16))
    for slots in (2, 1):
        out, _, _, _ = m.modulate_gemm_ring(xd, rs, shd, scd, qw, sfw, tw, chunk_rows=chunk, slots=slots)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_full.view(torch.int16)), slots
    sw, oqw, osfw, _ = _par.quantize_bf16(W)
    ref = _par.gemm_rows(oq, osf, s_g, oqw, osfw, sw, np.arange(M))
    ok, worst = oracle.gemm_tolerance_ok(out_f64(out_full), ref)
    assert ok, worst


@pytest.mark.parametrize("M,chunk,slots", [(300, 512, 1), (1000, 320, 1), (1000, 320, 2), (129, 64, 3)])
def test_ring_edge_shapes(m, M, chunk, slots):
    """One chunk larger than M, chunks that are not a multiple of the GEMM's
    256-row tile (outputs within tolerance, not bit-equal to the chained path
    there), chunks of 64 rows; slot bytes checked with one slot per chunk."""
    dev = device()
    K, N = 192, 272
    x = synth.normal_bf16(73, 0, (M, K), 1.0)
    sh = synth.normal_bf16(73, 1, (2, K), 0.1)
    sc = synth.normal_bf16(73, 2, (2, K), 0.1)
    W = synth.normal_bf16(73, 3, (N, K), 0.02)
    rs = [0, M // 3, M]
    xd, shd, scd = to_dev_u16(x), to_dev_u16(sh), to_dev_u16(sc)
    qw, sfw, tw = m.quantize_weight(to_dev_u16(W))
    seg = oracle.Segments(rs, sh, sc)
    s_g, oq, osf, _ = _par.modulate_quantize(x, seg, oracle.padded_rows(M))
    chunks = -(-M // chunk)
    out_all, ts, _, ring = m.modulate_gemm_ring(xd, rs, shd, scd, qw, sfw, tw, chunk_rows=chunk, slots=chunks)
    out, _, _, _ = m.modulate_gemm_ring(xd, rs, shd, scd, qw, sfw, tw, chunk_rows=chunk, slots=slots)
    torch.cuda.synchronize()
    assert host(ts)[0] == np.float32(s_g)
    check_slots(ring, chunk, M, K, oq, osf)
    assert torch.equal(out.view(torch.int16), out_all.view(torch.int16))
    sw, oqw, osfw, _ = _par.quantize_bf16(W)
    ref = _par.gemm_rows(oq, osf, s_g, oqw, osfw, sw, np.arange(M))
    ok, worst = oracle.gemm_tolerance_ok(out_f64(out), ref)
    assert ok, worst


def test_ring_qkv_canonical_19_chunks(m):
    """The QKV projection at M = 37,810 in 2048-row chunks (18 full chunks and
    a last one of 946 rows): each chunk's slot bytes against the oracle's
    QDATA/SFA rows (19 slots, none reused), the outputs equal to the chained
    path's in the 18 full chunks (no tile split along K there), the same with
    2 slots, and the checked rows (chunk bounds included) within the GEMM
    tolerance of the FP64 oracle."""
    w = synth.workload("qkv")
    dev = device()
    M, K, N, chunk = w.M, w.K, w.N, 2048
    x = w.x()
    rs, sh, sc = w.segments()
    W = w.weight()
    print(f"qkv ring: M={M} K={K} N={N} chunk {chunk}", flush=True)
    xd, shd, scd = to_dev_u16(x), to_dev_u16(sh), to_dev_u16(sc)
    qw, sfw, tw = m.quantize_weight(to_dev_u16(W))
    out19, ts, amax, ring = m.modulate_gemm_ring(xd, rs, shd, scd, qw, sfw, tw, chunk_rows=chunk, slots=19)
    torch.cuda.synchronize()
    seg = oracle.Segments(rs, sh, sc)
    s_g, oq, osf, _ = _par.modulate_quantize(x, seg, oracle.padded_rows(M))
    assert host(ts)[0] == np.float32(s_g)
    check_slots(ring, chunk, M, K, oq, osf)
    del ring
    print("slots byte-exact; chained path", flush=True)
    q, s, ts2, _ = m.modulate_quantize(xd, rs, shd, scd)
    chained = m.gemm(q, s, ts2, M, qw, sfw, tw)
    torch.cuda.synchronize()
    full = 18 * chunk
    assert torch.equal(out19[:full].view(torch.int16), chained[:full].view(torch.int16))
    del chained, q, s
    out2, _, _, _ = m.modulate_gemm_ring(xd, rs, shd, scd, qw, sfw, tw, chunk_rows=chunk, slots=2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out19.view(torch.int16))
    del out2
    print("outputs match; oracle rows", flush=True)
    rows = np.unique(np.concatenate([w.check_rows(48), np.array([2047, 2048, 36863, 36864, 37000, 37809])]))
    sw, oqw, osfw, _ = _par.quantize_bf16(W)
    ref = _par.gemm_rows(oq, osf, s_g, oqw, osfw, sw, rows)
    got = out_f64(out19[torch.from_numpy(rows).to(dev)])
    ok, worst = oracle.gemm_tolerance_ok(got, ref)
    print(f"qkv ring: worst err/bound {worst:.3g}", flush=True)
    assert ok, worst


def test_ring_argument_errors(m):
    dev = device()
    x = torch.zeros((128, 64), dtype=torch.bfloat16, device=dev)
    sh = torch.zeros((1, 64), dtype=torch.bfloat16, device=dev)
    seg, keep = m.make_segments([0, 128], sh, sh)
    ws = m.workspace(dev)
    f = torch.zeros(2, dtype=torch.float32, device=dev)
    ring = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
    qw = torch.zeros((64, 32), dtype=torch.uint8, device=dev)
    sfw = torch.zeros((64, 4), dtype=torch.uint8, device=dev)
    out = torch.zeros((128, 64), dtype=torch.bfloat16, device=dev)
    call = lambda slots, chunk, N=64: m.nvfp4_modulate_gemm_ring(  # noqa: E731
        x, 128, 64, 64, seg, ws, f, None, ring, slots, chunk, qw, sfw, f[1:], N, out, 64, None, 0)
    for slots, chunk, N in [(0, 64, 64), (65, 64, 64), (1, 100, 64), (1, 0, 64), (1, 64, 24)]:
        with pytest.raises(m.Nvfp4Error):
            call(slots, chunk, N)
    assert m.nvfp4_ring_slot_bytes(2048, 5376) == 2048 * (2688 + 336)
    assert m.nvfp4_ring_slot_bytes(100, 5376) == 0
    del keep
