"""The modulation and SwiGLU producers against the oracle: tensor scale bits,
QDATA and SFA byte for byte (padding rows included), at small and ragged
shapes, on adversarial values, and at the canonical 37,810-row sizes."""
import ctypes

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


def gpu_modulate(m, x, row_start, shift, scale, m_pad=None, ldx=None, single_pass=False):
    """Run the producer on the GPU (the two pass entry points, or the single
    launch); x may be given with a wider row stride."""
    M, D = x.shape
    if ldx is not None and ldx != D:
        wide = np.zeros((M, ldx), np.uint16)
        wide[:, :D] = x
        xd = to_dev_u16(wide)[:, :D]
    else:
        xd = to_dev_u16(x)
    q, s, ts, amax = m.modulate_quantize(xd, row_start, to_dev_u16(shift), to_dev_u16(scale), m_pad=m_pad,
                                         single_pass=single_pass)
    torch.cuda.synchronize()
    return host(ts)[0], host(q), host(s), host(amax)[0]


def check_modulate(m, x, row_start, shift, scale, m_pad=None, ldx=None):
    M = x.shape[0]
    m_pad = oracle.padded_rows(M) if m_pad is None else m_pad
    seg = oracle.Segments(row_start, shift, scale)
    s_g, q, s, amax = _par.modulate_quantize(x, seg, m_pad)
    for single in (False, True):
        gs, gq, gsf, gamax = gpu_modulate(m, x, row_start, shift, scale, m_pad, ldx, single)
        path = "single launch" if single else "two passes"
        assert np.float32(gamax).view(np.uint32) == np.float32(amax).view(np.uint32), (path, gamax, amax)
        assert np.float32(gs).view(np.uint32) == np.float32(s_g).view(np.uint32), (path, gs, s_g)
        assert np.array_equal(gsf, s), path + ": SFA " + str(first_mismatch(gsf, s))
        assert np.array_equal(gq, q), path + ": QDATA " + str(first_mismatch(gq, q))
    return s_g


def check_values(m, y):
    """Quantize a given bf16 tensor exactly: identity modulation (scale = +0,
    shift = -0) makes y = x for every non-NaN x."""
    D = y.shape[1]
    return check_modulate(m, y, np.array([0, y.shape[0]], np.int64), np.full((1, D), 0x8000, np.uint16),
                          np.zeros((1, D), np.uint16))


def bf16_np(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
def test_tiny_workload_byte_exact(m):
    w = synth.workload("tiny")
    x = w.x()
    rs, sh, sc = w.segments()
    check_modulate(m, x, rs, sh, sc)


@pytest.mark.parametrize("M,D,segs,ldx", [
    (1, 16, (0, 1), None),
    (63, 48, (0, 10, 63), None),
    (65, 528, (0, 1, 2, 64, 65), None),
    (130, 8208, (0, 70, 130), None),          # 1026 chunks per row: two chunks per thread
    (97, 5376, (0, 31, 97), 5392),            # strided rows
    (300, 256, tuple(range(0, 300, 20)) + (300,), None),   # 15 segments
    (40, 64, tuple(range(0, 16)) + (40,), None),            # 16 segments (the maximum)
    (21, 16400, (0, 5, 21), None),          # 1025 blocks per row: the single launch runs the two passes
    (769, 5376, (0, 500, 769), None),       # three-row groups, the last one partial
])
def test_ragged_shapes_and_segments(m, M, D, segs, ldx):
    rng = np.random.default_rng(M * 7 + D)
    x = bf16_np(rng.standard_normal((M, D)) * np.where(rng.random((M, D)) < 0.01, 100.0, 1.0))
    S = len(segs) - 1
    sh = bf16_np(0.1 * rng.standard_normal((S, D)))
    sc = bf16_np(0.1 * rng.standard_normal((S, D)))
    check_modulate(m, x, np.array(segs, np.int64), sh, sc, ldx=ldx)


def test_every_bf16_value_as_y(m):
    """All 65,280 non-NaN bf16 patterns (infinities included) as y, 16 per block."""
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = vals[(vals & 0x7FFF) <= 0x7F80]
    D = 512
    rows = (vals.size + D - 1) // D
    y = np.concatenate([vals, np.zeros(rows * D - vals.size, np.uint16)]).reshape(rows, D)
    check_values(m, y)
    # finite values only, clipped to a moderate maximum
    y2 = y.copy()
    big = (y2 & 0x7FFF) > 0x4700
    y2[big] = 0x4700 | (y2[big] & 0x8000)
    check_values(m, y2)


def test_subnormal_block_scales_and_saturation(m):
    """Blocks whose maximum is tiny next to the global one get E4M3-subnormal
    scales, where quotients exceed 6 and saturate."""
    D = 64
    rng = np.random.default_rng(31)
    y = bf16_np(np.array([rng.standard_normal(D) * 2.0 ** k for k in range(-24, 4)]))
    y[0, 0] = bf16_np([1000.0])[0]
    check_values(m, y)


def test_zero_tensor_gives_unit_scale(m):
    x = np.zeros((70, 32), np.uint16)
    sh = np.zeros((1, 32), np.uint16)
    sc = bf16_np(np.ones((1, 32)))
    s_g = check_modulate(m, x, np.array([0, 70]), sh, sc)
    assert s_g == 1.0


def test_signed_zeros_and_tiny_values(m):
    D = 32
    y = np.zeros((4, D), np.uint16)
    y[0, :] = 0x8000                       # -0 everywhere in a block next to a nonzero max
    y[0, 16] = 0x3F80
    y[1, :16] = 0x8001                     # smallest negative subnormal
    y[1, 16:] = 0x0001
    y[2, :] = bf16_np(np.linspace(-1e-3, 1e-3, D))
    y[3, 0] = 0x4000
    check_values(m, y)


def test_tiny_global_maximum_uses_exact_division(m):
    """A tensor whose maximum is so small that s_g is subnormal (outside the
    fast division range) still matches byte for byte."""
    rng = np.random.default_rng(33)
    y = bf16_np(rng.standard_normal((8, 64)) * 1e-38)
    check_values(m, y)
    y = bf16_np(rng.standard_normal((8, 64)) * 1e30)
    check_values(m, y)


@pytest.mark.parametrize("where", ["streamed", "held", "both"])
def test_nan_inputs_give_the_largest_nan_pattern(m, where):
    """NaN in x ([12000, 5376], 256 workgroups: rows of a workgroup's first
    groups are streamed in pass 1, the last ones held): the tensor maximum is
    the largest bf16 magnitude bit pattern of the device's own y (from the
    modulation step entry point on the same elements), in both launch forms,
    and every block packs to the NaN scale code with zero codes, as in the
    oracle.  Pass 1 takes the maximum of unrounded sums and reruns exactly
    when it meets a NaN, which this checks."""
    M, D = 12000, 5376
    x = synth.normal_bf16(81, 0, (M, D), 1.0)
    sh = synth.normal_bf16(81, 1, (2, D), 0.1)
    sc = synth.normal_bf16(81, 2, (2, D), 0.1)
    rs = [0, 7000, M]
    if where in ("streamed", "both"):
        x[1, 5] = 0x7FA1          # row 1: in workgroup 0's first (streamed) group
        x[4, 77] = 0xFFD3
    if where in ("held", "both"):
        x[M - 1, 4000] = 0x7FC9   # the last row: a register-held group
    seg_of = np.searchsorted(np.array(rs[1:]), np.arange(M), side="right")
    dev = device()
    y = torch.empty(M * D, dtype=torch.int16, device=dev)
    m.nvfp4_step_modulate(to_dev_u16(x.ravel()), to_dev_u16(sc[seg_of].ravel()), to_dev_u16(sh[seg_of].ravel()), y,
                          M * D)
    torch.cuda.synchronize()
    ymag = host(y).view(np.uint16) & 0x7FFF
    want_bits = np.uint32(ymag.max()) << 16
    assert (want_bits >> 16) > 0x7F80  # a NaN pattern
    seg = oracle.Segments(rs, sh, sc)
    _, oq, osf, _ = _par.modulate_quantize(x, seg, oracle.padded_rows(M))
    for single in (False, True):
        gs, gq, gsf, gamax = gpu_modulate(m, x, rs, sh, sc, single_pass=single)
        path = "single launch" if single else "two passes"
        assert np.float32(gamax).view(np.uint32) == want_bits, (path, hex(int(np.float32(gamax).view(np.uint32))))
        assert np.isnan(gs), path
        assert np.array_equal(gsf, osf) and (gsf[:M] == 0x7F).all(), path + ": SFA " + str(first_mismatch(gsf, osf))
        assert np.array_equal(gq, oq) and not gq.any(), path


def test_workspace_reuse_between_calls(m):
    """Calls in a row on one workspace, alternating the single launch and the
    two passes: each sees only its own tensor (the maxima differ).  The two
    passes leave their words at zero; the single launch tags its words with a
    tag of its own, so it needs no clearing either."""
    dev = device()
    rs = [0, 64]
    sh = torch.zeros((1, 64), dtype=torch.bfloat16, device=dev)
    sc = torch.zeros((1, 64), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(int(m.lib.nvfp4_absmax_workspace_bytes()), dtype=torch.uint8, device=dev)
    for single in (True, False, True, True):
        for val in (100.0, 2.0, 37.0):
            t = torch.full((64, 64), val, dtype=torch.bfloat16, device=dev)
            seg, keep = m.make_segments(rs, sh, sc)
            ts = torch.empty(1, dtype=torch.float32, device=dev)
            a = torch.empty(1, dtype=torch.float32, device=dev)
            q = torch.empty((64, 32), dtype=torch.uint8, device=dev)
            s = torch.empty((64, 4), dtype=torch.uint8, device=dev)
            if single:
                m.nvfp4_modulate_quantize(t, 64, 64, 64, seg, ws, ts, a, q, s, 64)
            else:
                m.nvfp4_modulate_absmax(t, 64, 64, 64, seg, ws, ts, a)
                m.nvfp4_modulate_pack(t, 64, 64, 64, seg, ts, q, s, 64)
            torch.cuda.synchronize()
            assert host(a)[0] == val
            assert host(ts)[0] == np.float32(val) / np.float32(2688.0)
            assert not host(ws)[:8].any()


def test_barrier_timeout_gives_nan_for_that_call_only(m):
    """The failure path of the single launches' grid barrier, forced from the
    host with a wait bound of 0 (every single launch gives up at once):
    modulation and SwiGLU calls complete with a NaN tensor scale and amax,
    scale code 0x7F in every block and zero codes (padding rows zero).  With
    the default bound restored, the next call on the same workspace is exact
    (every launch carries its own tag, so nothing of the abandoned one
    lingers)."""
    dev = device()
    rng = np.random.default_rng(7)
    M, D = 130, 256
    x = bf16_np(3 * rng.standard_normal((M, D)))
    rs = [0, 100, M]
    sh = bf16_np(0.1 * rng.standard_normal((2, D)))
    sc = bf16_np(0.1 * rng.standard_normal((2, D)))
    gu = bf16_np(2 * rng.standard_normal((M, 2 * D)))
    ws = torch.zeros(int(m.lib.nvfp4_absmax_workspace_bytes()), dtype=torch.uint8, device=dev)
    m_pad = oracle.padded_rows(M)
    seg, keep = m.make_segments(rs, to_dev_u16(sh), to_dev_u16(sc))

    def outputs():
        return (torch.zeros(1, dtype=torch.float32, device=dev), torch.zeros(1, dtype=torch.float32, device=dev),
                torch.full((m_pad, D // 2), 0x55, dtype=torch.uint8, device=dev),
                torch.full((m_pad, D // 16), 0x55, dtype=torch.uint8, device=dev))

    assert m.workspace_timeouts(ws) == 0
    previous = m.set_barrier_timeout_us(0)
    try:
        for i, kind in enumerate(("modulate", "swiglu", "modulate")):
            ts, a, q, s = outputs()
            if kind == "modulate":
                m.nvfp4_modulate_quantize(to_dev_u16(x), M, D, D, seg, ws, ts, a, q, s, m_pad)
            else:
                g = to_dev_u16(gu)
                m.nvfp4_swiglu_quantize(g, g.data_ptr() + 2 * D, M, D, 2 * D, ws, ts, a, q, s, m_pad)
            torch.cuda.synchronize()
            assert np.isnan(host(ts)[0]) and np.isnan(host(a)[0]), kind
            hs, hq = host(s), host(q)
            assert (hs[:M] == 0x7F).all() and not hs[M:].any(), kind
            assert not hq.any(), kind
            assert m.workspace_timeouts(ws) == i + 1, kind  # one count per abandoned launch
    finally:
        assert m.set_barrier_timeout_us(previous) == 0
    ts, a, q, s = outputs()
    m.nvfp4_modulate_quantize(to_dev_u16(x), M, D, D, seg, ws, ts, a, q, s, m_pad)
    torch.cuda.synchronize()
    s_g, oq, os_, amax = _par.modulate_quantize(x, oracle.Segments(rs, sh, sc), m_pad)
    assert host(ts)[0] == s_g and host(a)[0] == amax
    assert np.array_equal(host(s), os_), first_mismatch(host(s), os_)
    assert np.array_equal(host(q), oq), first_mismatch(host(q), oq)
    assert m.workspace_timeouts(ws) == 3  # sticky; a completed launch leaves it
    del keep


@pytest.mark.parametrize("kind", ["modulate", "plain", "swiglu"])
def test_helping_from_arrival_is_exact(m, kind):
    """With a help delay of 0 every workgroup, once it has reached the grid
    barrier, claims workgroups that have not arrived and computes their pass
    1 itself (the path taken when another kernel holds the CUs those
    workgroups need).  The maxima it stores are the ones those workgroups
    store, so every call is byte-exact, whether the shapes give each
    workgroup one row group or several, and with ragged segments."""
    rng = np.random.default_rng(23)
    previous = m.set_barrier_help_us(0)
    try:
        for M, D in ((1, 16), (700, 5376), (3001, 7168), (20011, 1056)):
            if kind == "swiglu":
                gu = bf16_np(2 * rng.standard_normal((M, 2 * D)))
                check_swiglu(m, gu)
            elif kind == "plain":
                check_plain(m, bf16_np(rng.standard_normal((M, D)) * np.exp(rng.standard_normal((M, 1)))))
            else:
                x = bf16_np(3 * rng.standard_normal((M, D)))
                rs = sorted({0, M, *(int(r) for r in rng.integers(0, M, 3))})
                ns = len(rs) - 1
                sh = bf16_np(0.1 * rng.standard_normal((ns, D)))
                sc = bf16_np(0.1 * rng.standard_normal((ns, D)))
                check_modulate(m, x, rs, sh, sc)
    finally:
        assert m.set_barrier_help_us(previous) == 0


def test_concurrent_single_launches_on_two_streams(m):
    """Two single-launch producers (modulation and SwiGLU) on two streams,
    enqueued behind a long matrix product on a third stream so that they
    start together and compete for the CUs.  Each needs all its workgroups'
    pass 1 before its barrier passes; workgroups that wait compute the pass 1
    of those that could not start, so both complete, exactly, and well inside
    the barrier's 1 s bound."""
    dev = device()
    rng = np.random.default_rng(19)
    M, D = 12000, 5376
    x = bf16_np(rng.standard_normal((M, D)))
    gu = bf16_np(2 * rng.standard_normal((M // 4, 2 * 3584)))
    rs = [0, 9000, M]
    sh = bf16_np(0.1 * rng.standard_normal((2, D)))
    sc = bf16_np(0.1 * rng.standard_normal((2, D)))
    want_mod = _par.modulate_quantize(x, oracle.Segments(rs, sh, sc), oracle.padded_rows(M))
    want_sw = _par.swiglu_quantize(gu, oracle.padded_rows(M // 4))
    xd, gud, shd, scd = to_dev_u16(x), to_dev_u16(gu), to_dev_u16(sh), to_dev_u16(sc)
    big = torch.randn((8192, 8192), device=dev)
    s0, s1, s2 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(s0):
            for _ in range(4):
                big = big @ big * 1e-4
        events = []
        with torch.cuda.stream(s1):
            a1 = torch.cuda.Event(enable_timing=True)
            b1 = torch.cuda.Event(enable_timing=True)
            a1.record(s1)
            got_mod = m.modulate_quantize(xd, rs, shd, scd, stream=s1)
            b1.record(s1)
        with torch.cuda.stream(s2):
            a2 = torch.cuda.Event(enable_timing=True)
            b2 = torch.cuda.Event(enable_timing=True)
            a2.record(s2)
            got_sw = m.swiglu_quantize(gud, stream=s2)
            b2.record(s2)
        torch.cuda.synchronize()
        ms = (a1.elapsed_time(b1), a2.elapsed_time(b2))
        print(f"rep {rep}: {ms[0]:.2f} ms, {ms[1]:.2f} ms", flush=True)
        for (gq, gs, gts, gamax), (s_g, q, s, amax), name in ((got_mod, want_mod, "modulation"),
                                                             (got_sw, want_sw, "swiglu")):
            assert host(gts)[0] == s_g and host(gamax)[0] == amax, (rep, name)
            assert np.array_equal(host(gs), s) and np.array_equal(host(gq), q), (rep, name)
        assert max(ms) < 500.0, ms


def test_non_default_stream(m):
    w = synth.workload("tiny")
    x = w.x()
    rs, sh, sc = w.segments()
    seg = oracle.Segments(rs, sh, sc)
    s_g, q, s, _ = oracle.modulate_quantize(x, seg)
    st = torch.cuda.Stream()
    xd, shd, scd = to_dev_u16(x), to_dev_u16(sh), to_dev_u16(sc)
    torch.cuda.synchronize()
    for single in (False, True):
        with torch.cuda.stream(st):
            gq, gs, gts, _ = m.modulate_quantize(xd, rs, shd, scd, stream=st, single_pass=single)
        st.synchronize()
        assert np.array_equal(host(gq), q) and np.array_equal(host(gs), s)
        assert host(gts)[0] == s_g


def test_two_streams_get_their_own_workspaces(m):
    """The convenience calls on two streams, enqueued back to back with no
    synchronization between them (the two-pass path, which has no grid
    barrier): each stream has its own workspace, so the two tensors' maxima
    never mix; both results match the oracle."""
    dev = device()
    rng = np.random.default_rng(11)
    M, D = 3000, 512
    xs = [bf16_np(a * rng.standard_normal((M, D))) for a in (1.0, 40.0)]
    rs = [0, 1000, M]
    sh = bf16_np(0.1 * rng.standard_normal((2, D)))
    sc = bf16_np(0.1 * rng.standard_normal((2, D)))
    seg = oracle.Segments(rs, sh, sc)
    want = [_par.modulate_quantize(x, seg, oracle.padded_rows(M)) for x in xs]
    xd = [to_dev_u16(x) for x in xs]
    shd, scd = to_dev_u16(sh), to_dev_u16(sc)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    assert m.workspace(dev, streams[0]).data_ptr() != m.workspace(dev, streams[1]).data_ptr()
    for rep in range(3):
        got = []
        for x, st in zip(xd, streams):
            with torch.cuda.stream(st):
                got.append(m.modulate_quantize(x, rs, shd, scd, stream=st, single_pass=False))
        torch.cuda.synchronize()
        for (gq, gs, gts, gamax), (s_g, q, s, amax) in zip(got, want):
            assert host(gts)[0] == s_g and host(gamax)[0] == amax, rep
            assert np.array_equal(host(gs), s) and np.array_equal(host(gq), q), rep


def test_single_launch_without_amax_output(m):
    """nvfp4_modulate_quantize with amax_out = NULL writes the same bytes."""
    w = synth.workload("tiny")
    x = w.x()
    rs, sh, sc = w.segments()
    s_g, q, s, _ = oracle.modulate_quantize(x, oracle.Segments(rs, sh, sc))
    dev = device()
    seg, keep = m.make_segments(rs, to_dev_u16(sh), to_dev_u16(sc))
    xd = to_dev_u16(x)
    mp = oracle.padded_rows(w.M)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    qd = torch.full((mp, w.K // 2), 0xAB, dtype=torch.uint8, device=dev)
    sd = torch.full((mp, w.K // 16), 0xAB, dtype=torch.uint8, device=dev)
    m.nvfp4_modulate_quantize(xd, w.M, w.K, w.K, seg, m.workspace(dev), ts, None, qd, sd, mp)
    torch.cuda.synchronize()
    assert host(ts)[0] == s_g and np.array_equal(host(qd), q) and np.array_equal(host(sd), s)
    del keep


def test_single_launch_streams_and_holds_rows(m):
    """A tensor large enough that every workgroup of the single launch streams
    rows again in its second pass, besides the rows it holds in registers and
    LDS (60,000 x 1,024), with 16 segments whose boundaries the reversed second
    pass crosses."""
    rng = np.random.default_rng(77)
    M, D = 60000, 1024
    x = bf16_np(rng.standard_normal((M, D)) * np.where(rng.random((M, D)) < 0.001, 50.0, 1.0))
    segs = np.array([0, 1, 17, 1000, 4095, 4096, 9000, 15000, 22222, 30000, 30001, 41000, 50000, 55555, 59000,
                     59999, 60000], np.int64)
    S = segs.size - 1
    sh = bf16_np(0.1 * rng.standard_normal((S, D)))
    sc = bf16_np(0.1 * rng.standard_normal((S, D)))
    check_modulate(m, x, segs, sh, sc)


@pytest.mark.parametrize("kind", ["shift", "scale", "segment", "late", "inf_times_zero"])
def test_pass1_maximum_from_any_column_segment_or_row(m, kind):
    """Tensor maxima that a bound on |y| from |x| alone would miss, in rows the
    single launch streams in pass 1 ([126976, 1024]: 31 row groups of 16 rows
    per workgroup, the first 20 streamed, two per iteration): a maximum made by
    one column's shift, by one column's scale, by a row of the second segment
    whose pass-1 partner row is in the first, by an outlier in a workgroup's
    last streamed pair, and a NaN from x = Inf times bf16(scale+1) = 0.  Amax
    bits and tensor scale against the oracle in both launch forms; all bytes
    for the segment case."""
    M, D, B0 = 126976, 1024, 41080
    x = synth.normal_bf16(91, 0, (M, D), 1.0)
    sh = synth.normal_bf16(91, 1, (2, D), 0.1)
    sc = synth.normal_bf16(91, 2, (2, D), 0.1)
    rs = [0, B0, M]
    if kind == "shift":
        sh[1, 700] = bf16_np(1000.0)
    elif kind == "scale":
        sc[0, 33] = bf16_np(300.0)
    elif kind == "segment":
        # row 45091 = group 11 of workgroup 2 (row 3 of 16); its pair row in
        # group 10, 40995, lies before the segment boundary
        sc[1, 517] = bf16_np(20.0)
        x[B0:, 517] = bf16_np(0.01)
        x[45091, 517] = bf16_np(4.0)
    elif kind == "late":
        x[77829, 100] = bf16_np(250.0)   # group 19 of workgroup 0
    else:
        sc[0, 900] = bf16_np(-1.0)
        x[41015, 900] = 0x7F80           # group 10 of workgroup 3
    print(f"pass-1 maximum case {kind}", flush=True)
    if kind == "segment":
        check_modulate(m, x, np.array(rs, np.int64), sh, sc)
        return
    seg = oracle.Segments(rs, sh, sc)
    amax = np.float32(_par.amax_merge(_par._map(lambda r: oracle.modulate_amax_rows(x, seg, *r),
                                                 _par._ranges(M, 4 * _par.WORKERS))))
    s_g = np.float32(oracle.tensor_scale(float(amax)))
    if kind == "inf_times_zero":
        assert (amax.view(np.uint32) >> 16) > 0x7F80
    for single in (False, True):
        gs, _, _, gamax = gpu_modulate(m, x, rs, sh, sc, single_pass=single)
        path = "single launch" if single else "two passes"
        assert np.float32(gamax).view(np.uint32) == amax.view(np.uint32), (path, gamax, amax)
        assert np.float32(gs).view(np.uint32) == s_g.view(np.uint32) or (np.isnan(gs) and np.isnan(s_g)), path


@pytest.mark.parametrize("M", [12001, 769])
@pytest.mark.parametrize("amax", [2688.0, 13.125])
def test_tensor_scales_with_short_binary_expansions(m, amax, M):
    """Tensor maxima that make s_g a power of two (2688: s_g = 1, so every
    divisor is an E4M3 value and many quotients fall exactly on E2M1
    midpoints) or a short binary fraction (13.125 = 210/16: s_g = 2^-8 * 5/4),
    with ragged row counts that leave rows past M in the last row group.  Bytes
    against the oracle for the modulation producer (both launch forms) and the
    plain quantizer."""
    D = 5376
    x = synth.normal_bf16(97, 0, (M, D), 1.0)
    x[M // 2, 1234] = bf16_np(amax)
    print(f"short-expansion scales: amax {amax} M {M}", flush=True)
    s_g = check_values(m, x)
    assert s_g in (np.float32(1.0), np.float32(2.0 ** -8 * 1.25))
    check_plain(m, x)


def test_weight_prepack_matches_oracle_quantizer(m):
    w = synth.workload("tiny").weight()
    sw, qw, sfw, _ = _par.quantize_bf16(w)
    gq, gs, gts = m.quantize_weight(to_dev_u16(w))
    torch.cuda.synchronize()
    assert host(gts)[0] == sw
    assert np.array_equal(host(gq), qw) and np.array_equal(host(gs), sfw)


# --------------------------------------------------------------------------
# Plain quantizer (no modulation)
# --------------------------------------------------------------------------
def check_plain(m, y, m_pad=None, nan_ok=False):
    M = y.shape[0]
    m_pad = oracle.padded_rows(M) if m_pad is None else m_pad
    s_g, q, s, amax = _par.quantize_bf16(y, m_pad)
    gq, gs, gts, gamax = m.quantize(to_dev_u16(y), m_pad=m_pad)
    torch.cuda.synchronize()
    ga, gt = np.float32(host(gamax)[0]), np.float32(host(gts)[0])
    if nan_ok and np.isnan(amax):
        assert np.isnan(ga) and np.isnan(gt)
        # the maximum is the largest magnitude bit pattern, NaN payload included
        assert (ga.view(np.uint32) >> 16) & 0x7FFF == (np.float32(amax).view(np.uint32) >> 16) & 0x7FFF
    else:
        assert ga.view(np.uint32) == np.float32(amax).view(np.uint32) and gt == np.float32(s_g)
    assert np.array_equal(host(gs), s), "SFA " + str(first_mismatch(host(gs), s))
    assert np.array_equal(host(gq), q), "QDATA " + str(first_mismatch(host(gq), q))


@pytest.mark.parametrize("M,D", [(1, 16), (63, 48), (769, 5376), (130, 8208), (21, 16400), (300, 7168)])
def test_plain_quantizer_shapes(m, M, D):
    rng = np.random.default_rng(M * 3 + D)
    y = bf16_np(rng.standard_normal((M, D)) * np.where(rng.random((M, D)) < 0.01, 100.0, 1.0))
    check_plain(m, y)


def test_plain_quantizer_every_bf16_value_and_nan(m):
    """All 65,536 bf16 patterns, NaN included: the plain quantizer passes NaN
    through, the maximum is NaN and every block gets the NaN scale code."""
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    y = vals.reshape(128, 512)
    check_plain(m, y, nan_ok=True)
    finite = vals[(vals & 0x7FFF) < 0x7F80]
    D = 512
    rows = (finite.size + D - 1) // D
    y2 = np.concatenate([finite, np.zeros(rows * D - finite.size, np.uint16)]).reshape(rows, D)
    check_plain(m, y2)


def test_plain_quantizer_attention_output_canonical(m):
    """The attention-output activation [37810, 7168] through the plain
    quantizer, every row byte-exact."""
    w = synth.workload("attn_out")
    x = w.x()
    print(f"attn_out activation {x.shape}", flush=True)
    check_plain(m, x)


# --------------------------------------------------------------------------
# SwiGLU producer
# --------------------------------------------------------------------------
def check_swiglu(m, gu, m_pad=None):
    M = gu.shape[0]
    m_pad = oracle.padded_rows(M) if m_pad is None else m_pad
    s_g, q, s, amax = _par.swiglu_quantize(gu, m_pad)
    for combined in (True, False):
        gq, gs, gts, gamax = m.swiglu_quantize(to_dev_u16(gu), m_pad=m_pad, combined=combined)
        torch.cuda.synchronize()
        path = "one call" if combined else "two calls"
        assert host(gamax)[0] == amax and host(gts)[0] == s_g, path
        assert np.array_equal(host(gs), s), path + ": SFA " + str(first_mismatch(host(gs), s))
        assert np.array_equal(host(gq), q), path + ": QDATA " + str(first_mismatch(host(gq), q))


# F = 16400: more than 1024 blocks per row, so pack threads take two blocks
@pytest.mark.parametrize("M,F", [(1, 16), (77, 48), (200, 512), (65, 8208), (5, 16400)])
def test_swiglu_small_shapes(m, M, F):
    rng = np.random.default_rng(M + F)
    gu = bf16_np(3 * rng.standard_normal((M, 2 * F)))
    check_swiglu(m, gu)


def test_swiglu_separate_gate_and_up_pointers(m):
    """gate and up as two separate [M, F] tensors with their own stride."""
    rng = np.random.default_rng(41)
    M, F = 90, 96
    g = bf16_np(2 * rng.standard_normal((M, F)))
    u = bf16_np(rng.standard_normal((M, F)))
    gu = np.concatenate([g, u], axis=1)
    s_g, q, s, _ = _par.swiglu_quantize(gu, 128)
    dev = device()
    gd, ud = to_dev_u16(g), to_dev_u16(u)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    qd = torch.empty((128, F // 2), dtype=torch.uint8, device=dev)
    sd = torch.empty((128, F // 16), dtype=torch.uint8, device=dev)
    m.nvfp4_swiglu_absmax(gd, ud, M, F, F, m.workspace(dev), ts)
    m.nvfp4_swiglu_pack(gd, ud, M, F, F, ts, qd, sd, 128)
    torch.cuda.synchronize()
    assert host(ts)[0] == s_g and np.array_equal(host(qd), q) and np.array_equal(host(sd), s)


# --------------------------------------------------------------------------
# canonical sizes
# --------------------------------------------------------------------------
def test_producer_canonical_37810_rows_byte_exact(m):
    """The 37,810 x 5,376 producer workload, two segments, every row."""
    w = synth.workload("producer")
    x = w.x()
    rs, sh, sc = w.segments()
    print(f"producer workload {x.shape}", flush=True)
    s_g = check_modulate(m, x, rs, sh, sc)
    assert s_g > 0


def test_fc1_producer_canonical_37810_rows_byte_exact(m):
    """The FC1 projection's producer: the same 37,810 x 5,376 activation with
    the FC1 shift/scale (their own seed), every row, both launch forms."""
    w = synth.workload("fc1")
    x = w.x()
    rs, sh, sc = w.segments()
    print(f"fc1 producer workload {x.shape}", flush=True)
    s_g = check_modulate(m, x, rs, sh, sc)
    assert s_g > 0


def test_swiglu_canonical_37810_rows_byte_exact(m):
    """The 37,810 x 2*14,336 FC2 SwiGLU producer: tensor scale, QDATA and SFA
    of every row (padding included), in both launch forms."""
    w = synth.workload("fc2")
    gu = w.gate_up()
    print(f"swiglu workload {gu.shape}", flush=True)
    check_swiglu(m, gu)


# Inputs past 4 GiB: byte offsets beyond 2^32, where the producers leave the
# single launch and 32-bit offsets for the two passes with 64-bit offsets.
# The rows repeat a seeded block of 61 rows (a period that no tiling of the
# kernels divides), built on the device; the oracle runs on the block.
_P = 61


def _tiled_dev(block, M):
    b = to_dev_u16(block)
    return b.repeat(-(-M // _P), 1)[:M].contiguous()


def _rows_past_4gib(c, M, row_bytes, must):
    """Sampled rows over the whole range, most of them past byte 2^32."""
    first = -(-(1 << 32) // row_bytes)
    lo = synth.sample_rows(c, first, 48, must=[r for r in must if r < first])
    hi = first + synth.sample_rows(c + 1, M - first, 160, must=[r - first for r in must if r >= first])
    return np.unique(np.concatenate([lo, hi]))


def test_modulation_and_plain_inputs_past_4_gib(m):
    """x [400,000, 5,376] bf16 (4.30 GB), two segments: tensor scale, QDATA and
    SFA of sampled rows (incl. both sides of the segment boundary and the last
    row) and every padding row, for the modulation producer and the plain
    quantizer."""
    M, D = 400_000, 5376
    assert (M - 1) * D * 2 >= 1 << 32
    boundary = 250_001
    block = synth.add_outliers_t3(synth.normal_bf16(40, 0, (_P, D), 1.0), 40, 0.001, 20.0)
    sh = synth.normal_bf16(41, 1, (2, D), 0.1)
    sc = synth.normal_bf16(41, 2, (2, D), 0.1)
    rs = [0, boundary, M]
    print(f"x [{M}, {D}] tiled from {_P} rows on the device", flush=True)
    x = _tiled_dev(block, M)
    q, s, ts, amax = m.modulate_quantize(x, rs, to_dev_u16(sh), to_dev_u16(sc))
    torch.cuda.synchronize()
    # every row phase occurs in both segments, so the global maximum is the
    # block's maximum under either segment's parameters
    seg2 = oracle.Segments([0, _P, 2 * _P], sh, sc)
    oamax = oracle.modulate_amax_rows(np.concatenate([block, block]), seg2, 0, 2 * _P)
    s_g = np.float32(oracle.tensor_scale(oamax))
    assert np.float32(host(amax)[0]).view(np.uint32) == np.float32(oamax).view(np.uint32)
    assert host(ts)[0].view(np.uint32) == s_g.view(np.uint32)
    rows = _rows_past_4gib(42, M, D * 2, [0, boundary - 1, boundary, M - 1])
    n0 = int(np.searchsorted(rows, boundary))
    assert 0 < n0 < rows.size
    oq, os_ = oracle.modulate_pack_rows(block[rows % _P], oracle.Segments([0, n0, rows.size], sh, sc), s_g,
                                        0, rows.size)
    ridx = torch.from_numpy(rows).to(x.device)
    gq, gs = host(q[ridx]), host(s[ridx])
    assert np.array_equal(gs, os_), first_mismatch(gs, os_)
    assert np.array_equal(gq, oq), first_mismatch(gq, oq)
    assert not host(q[M:]).any() and not host(s[M:]).any()
    del q, s

    print("plain quantizer on the same x", flush=True)
    q, s, ts, amax = m.quantize(x)
    torch.cuda.synchronize()
    pamax = oracle.bf16_amax(block)
    ps_g = np.float32(oracle.tensor_scale(pamax))
    assert host(ts)[0].view(np.uint32) == ps_g.view(np.uint32)
    oq, os_ = oracle.bf16_pack_rows(block[rows % _P], ps_g, 0, rows.size)
    gq, gs = host(q[ridx]), host(s[ridx])
    assert np.array_equal(gs, os_), first_mismatch(gs, os_)
    assert np.array_equal(gq, oq), first_mismatch(gq, oq)
    assert not host(q[M:]).any() and not host(s[M:]).any()


def test_swiglu_input_past_4_gib(m):
    """gate/up [80,000, 2*14,336] bf16 (4.59 GB; the pack pass's 64-bit offset
    variant): tensor scale, QDATA and SFA of sampled rows and every padding
    row."""
    M, F = 80_000, 14_336
    assert (M - 1) * 2 * F * 2 >= 1 << 32
    block = synth.normal_bf16(43, 0, (_P, 2 * F), 1.0)
    print(f"gate/up [{M}, {2 * F}] tiled from {_P} rows on the device", flush=True)
    gu = _tiled_dev(block, M)
    q, s, ts, amax = m.swiglu_quantize(gu)
    torch.cuda.synchronize()
    oamax = oracle.swiglu_amax_rows(block, 0, _P)
    s_g = np.float32(oracle.tensor_scale(oamax))
    assert np.float32(host(amax)[0]).view(np.uint32) == np.float32(oamax).view(np.uint32)
    assert host(ts)[0].view(np.uint32) == s_g.view(np.uint32)
    rows = _rows_past_4gib(44, M, 4 * F, [0, M - 1])
    oq, os_ = oracle.swiglu_pack_rows(block[rows % _P], s_g, 0, rows.size)
    ridx = torch.from_numpy(rows).to(gu.device)
    gq, gs = host(q[ridx]), host(s[ridx])
    assert np.array_equal(gs, os_), first_mismatch(gs, os_)
    assert np.array_equal(gq, oq), first_mismatch(gq, oq)
    assert not host(q[M:]).any() and not host(s[M:]).any()


def test_conveniences_under_graph_capture_replay_like_eager(m):
    """modulate_quantize, swiglu_quantize and quantize with their defaults,
    captured into a HIP graph, take their two-launch forms (the single
    launch's barrier tag comes from the host and would replay): four replays
    with new inputs copied into the captured input buffers, each byte-equal
    to the same conveniences run eagerly (single launches) in between."""
    dev = device()
    M, D, F = 3000, 2048, 1024
    rs = [0, 1700, M]
    sh = to_dev_u16(synth.normal_bf16(61, 1, (2, D), 0.1))
    sc = to_dev_u16(synth.normal_bf16(61, 2, (2, D), 0.1))
    x = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    gu = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=dev)

    def fill(seed):
        x.copy_(to_dev_u16(synth.add_outliers_t3(synth.normal_bf16(seed, 0, (M, D), 1.0), seed, 0.001, 20.0)))
        gu.copy_(to_dev_u16(synth.normal_bf16(seed, 3, (M, 2 * F), 1.0)))

    def run_all():
        return (m.modulate_quantize(x, rs, sh, sc), m.swiglu_quantize(gu), m.quantize(x))

    def bytes_of(res):
        return [tuple(host(t).tobytes() for t in r) for r in res]

    fill(300)
    run_all()  # eager first: workspaces of this stream and the library's tables
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # captured on the graph's own stream, the current one inside
        captured = run_all()
    torch.cuda.synchronize()
    for rep, seed in enumerate((301, 302, 303, 304)):
        print(f"replay {rep} with input seed {seed}", flush=True)
        fill(seed)
        torch.cuda.synchronize()
        want = bytes_of(run_all())  # eager single launches between the replays
        for r in captured:
            for t in r:
                t.fill_(0x5A if t.dtype == torch.uint8 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bytes_of(captured)
        for name, gw, ww in zip(("modulation", "swiglu", "plain"), got, want):
            for part, a, b in zip(("qdata", "sfa", "tensor scale", "amax"), gw, ww):
                assert a == b, (rep, name, part)
