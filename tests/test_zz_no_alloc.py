"""nvfp4_modulate_quantize_noalloc against nvfp4_modulate_quantize: the same
tensor scale, amax, QDATA and SFA bytes, through the C ABI, on consecutive
calls (the second on a smaller input, so that words left by the first call in
the shared scratch would show), on the two-pass form it falls back to for
rows wider than 16,384 values, and captured into a graph: every replay, with
new contents in the same input buffer and eager work and synchronizations
between the replays, matches the workspace entry point run eagerly."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import device, first_mismatch, host, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import nvfp4_activation_quantization_segment_amd as pkg

    device()
    return pkg


def _inputs(c, M, D, cut):
    x = synth.add_outliers_t3(synth.normal_bf16(c, 0, (M, D), 1.0), c, 0.001, 20.0)
    sh = synth.normal_bf16(c, 1, (2, D), 0.1)
    sc = synth.normal_bf16(c, 2, (2, D), 0.1)
    return to_dev_u16(x), [0, cut, M], to_dev_u16(sh), to_dev_u16(sc)


def _outputs(dev, M_pad, D):
    return (torch.full((1,), float("nan"), dtype=torch.float32, device=dev),
            torch.full((1,), float("nan"), dtype=torch.float32, device=dev),
            torch.full((M_pad, D // 2), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((M_pad, D // 16), 0x5A, dtype=torch.uint8, device=dev))


def _run_both(m, x, rs, sh, sc):
    M, D = x.shape
    M_pad = m.padded_rows(M)
    dev = x.device
    seg, keep = m.make_segments(rs, sh, sc)
    ts0, am0, q0, s0 = _outputs(dev, M_pad, D)
    m.nvfp4_modulate_quantize(x, M, D, x.stride(0), seg, m.workspace(dev), ts0, am0, q0, s0, M_pad)
    ts1, am1, q1, s1 = _outputs(dev, M_pad, D)
    m.nvfp4_modulate_quantize_noalloc(x, M, D, x.stride(0), seg, ts1, am1, q1, s1, M_pad)
    torch.cuda.synchronize()
    del keep
    return (host(ts0), host(am0), host(q0), host(s0)), (host(ts1), host(am1), host(q1), host(s1))


def _same(ref, got, what):
    assert ref[0].view(np.uint32)[0] == got[0].view(np.uint32)[0], (what, "tensor scale", ref[0], got[0])
    assert ref[1].view(np.uint32)[0] == got[1].view(np.uint32)[0], (what, "amax", ref[1], got[1])
    assert np.array_equal(ref[3], got[3]), (what, "SFA", first_mismatch(got[3], ref[3]))
    assert np.array_equal(ref[2], got[2]), (what, "QDATA", first_mismatch(got[2], ref[2]))


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls(m):
    cases = [(61, 4000, 5376, 3100), (62, 700, 1024, 300)]   # the second call is smaller
    for c, M, D, cut in cases:
        print(f"noalloc vs workspace: M={M} D={D} segments [0,{cut},{M}]", flush=True)
        x, rs, sh, sc = _inputs(c, M, D, cut)
        ref, got = _run_both(m, x, rs, sh, sc)
        assert np.isfinite(ref[0][0]) and ref[0][0] > 0
        _same(ref, got, f"M={M} D={D}")


def test_noalloc_two_pass_form_for_wide_rows(m):
    """D = 16,400 (more than 1,024 blocks per row): both entry points enqueue the
    two passes, whose maximum and counter words the no-allocation call also
    keeps in the scratch."""
    M, D = 130, 16400
    print(f"noalloc two-pass form: M={M} D={D}", flush=True)
    x, rs, sh, sc = _inputs(63, M, D, 77)
    ref, got = _run_both(m, x, rs, sh, sc)
    _same(ref, got, f"M={M} D={D}")


def test_noalloc_rejects_bad_arguments_before_launch(m):
    """Argument errors return synchronously, as for the workspace entry point."""
    dev = device()
    x = torch.zeros((64, 48), dtype=torch.bfloat16, device=dev)
    sh = torch.zeros((1, 48), dtype=torch.bfloat16, device=dev)
    seg, keep = m.make_segments([0, 64], sh, sh)
    ts, am, q, s = _outputs(dev, 64, 48)
    with pytest.raises(m.Nvfp4Error):
        m.nvfp4_modulate_quantize_noalloc(x, 64, 40, 48, seg, ts, am, q, s, 64)   # D % 16 != 0
    with pytest.raises(m.Nvfp4Error):
        m.nvfp4_modulate_quantize_noalloc(x, 64, 48, 48, seg, ts, am, q, s, 32)   # M_pad too small
    bad, keep2 = m.make_segments([0, 63], sh, sh)
    with pytest.raises(m.Nvfp4Error):
        m.nvfp4_modulate_quantize_noalloc(x, 64, 48, 48, bad, ts, am, q, s, 64)   # rows do not end at M
    del keep, keep2


def test_noalloc_graph_replays_match_eager(m):
    dev = device()
    M, D, cut = 12000, 5376, 7000  # about 16 row groups per workgroup: both streamed and held rows
    M_pad = m.padded_rows(M)
    sh = to_dev_u16(synth.normal_bf16(91, 1, (2, D), 0.1))
    sc = to_dev_u16(synth.normal_bf16(91, 2, (2, D), 0.1))
    seg, keep = m.make_segments([0, cut, M], sh, sc)
    x = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    q = torch.empty((M_pad, D // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((M_pad, D // 16), dtype=torch.uint8, device=dev)

    def fill(seed):
        x.copy_(to_dev_u16(synth.add_outliers_t3(synth.normal_bf16(seed, 0, (M, D), 1.0), seed, 0.001, 20.0)))

    def eager_reference():
        rts = torch.empty(1, dtype=torch.float32, device=dev)
        ram = torch.empty(1, dtype=torch.float32, device=dev)
        rq = torch.empty((M_pad, D // 2), dtype=torch.uint8, device=dev)
        rs = torch.empty((M_pad, D // 16), dtype=torch.uint8, device=dev)
        m.nvfp4_modulate_quantize(x, M, D, D, seg, m.workspace(dev), rts, ram, rq, rs, M_pad)
        torch.cuda.synchronize()
        return host(rts), host(ram), host(rq), host(rs)

    fill(100)
    # an eager call first: the scratch address and the grid size are looked up outside capture
    m.nvfp4_modulate_quantize_noalloc(x, M, D, D, seg, ts, amax, q, s, M_pad)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # captured on the graph's own stream, the current one inside
        m.nvfp4_modulate_quantize_noalloc(x, M, D, D, seg, ts, amax, q, s, M_pad)
    torch.cuda.synchronize()
    for rep, seed in enumerate((101, 102, 103, 104)):
        print(f"replay {rep} with input seed {seed}", flush=True)
        fill(seed)
        torch.cuda.synchronize()
        want = eager_reference()  # eager work between the replays
        q.fill_(0xA5)
        s.fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        got = (host(ts), host(amax), host(q), host(s))
        assert got[0].view(np.uint32)[0] == want[0].view(np.uint32)[0], (rep, "tensor scale")
        assert got[1].view(np.uint32)[0] == want[1].view(np.uint32)[0], (rep, "amax")
        assert np.array_equal(got[3], want[3]), (rep, "SFA", first_mismatch(got[3], want[3]))
        assert np.array_equal(got[2], want[2]), (rep, "QDATA", first_mismatch(got[2], want[2]))
    del g, keep
