"""Seeded random sweeps over the shapes, strides, segment tables and value
ranges the entry points accept, each case against the oracle: the producers
byte for byte (single launch and two passes), the GEMM within its tolerance
(with and without the K-split workspace).  The cases are drawn once from a
fixed seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import oracle
from tests import _par
from tests.gpu_util import device, to_dev
from tests.test_gpu_producer import bf16_np, check_modulate, check_plain, check_swiglu
from tests.test_gpu_gemm import check, gpu_gemm, oracle_quantized, out_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import nvfp4_activation_quantization_segment_amd as pkg

    device()
    return pkg


def _values(rng, shape):
    """Normal values times a per-row log-normal magnitude, with some exact zeros."""
    a = rng.standard_normal(shape) * np.exp(1.5 * rng.standard_normal((shape[0], 1)))
    a[rng.random(shape) < 0.02] = 0.0
    return bf16_np(a)


def _producer_cases(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 70)), int(rng.integers(70, 3000))]))
        D = 16 * int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 700))]))
        pad = 8 * int(rng.integers(0, 3))
        cases.append((M, D, pad, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("M,D,pad,seed", _producer_cases(101, 40))
def test_modulation_sweep(m, M, D, pad, seed):
    rng = np.random.default_rng(seed)
    x = _values(rng, (M, D))
    cuts = sorted(int(c) for c in rng.integers(1, M, int(rng.integers(0, 4)))) if M > 1 else []
    rs = [0] + sorted(set(cuts)) + [M]
    ns = len(rs) - 1
    sh = bf16_np(rng.standard_normal((ns, D)) * 0.5)
    sc = bf16_np(rng.standard_normal((ns, D)) * 0.5)
    check_modulate(m, x, rs, sh, sc, ldx=D + pad)


@pytest.mark.parametrize("M,D,pad,seed", _producer_cases(202, 24))
def test_plain_quantizer_sweep(m, M, D, pad, seed):
    rng = np.random.default_rng(seed)
    check_plain(m, _values(rng, (M, D)), m_pad=oracle.padded_rows(M) + 64 * int(rng.integers(0, 2)))


@pytest.mark.parametrize("M,D,pad,seed", _producer_cases(303, 24))
def test_swiglu_sweep(m, M, D, pad, seed):
    rng = np.random.default_rng(seed)
    gu = bf16_np(rng.standard_normal((M, 2 * D)) * 2.0)
    check_swiglu(m, gu)


def _gemm_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        N = 16 * int(rng.integers(1, 70))
        K = 64 * int(rng.integers(1, 40))
        out.append((M, N, K, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("M,N,K,seed", _gemm_cases(404, 30))
def test_gemm_sweep(m, M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = _values(rng, (M, K))
    w = bf16_np(0.05 * rng.standard_normal((N, K)))
    m_pad = oracle.padded_rows(M)
    sa, qa, sfa, sw, qw, sfw = oracle_quantized(a, w, m_pad)
    ref = _par.gemm_rows(qa, sfa, sa, qw, sfw, sw, np.arange(M))
    out = gpu_gemm(m, sa, qa, sfa, sw, qw, sfw, M)
    check(ref, out_f64(out), f"{M}x{N}x{K}")
    # the workspace form (K-split of a short last wave where the plan has one)
    dev = device()
    nbytes = int(m.nvfp4_gemm_workspace_bytes(M, N, K))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    out2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    m.nvfp4_gemm_ws(to_dev(qa), to_dev(sfa), to_dev(np.array([sa], np.float32)), M, m_pad, to_dev(qw),
                    to_dev(sfw), to_dev(np.array([sw], np.float32)), N, K, out2, N, ws, nbytes)
    torch.cuda.synchronize()
    check(ref, out_f64(out2), f"{M}x{N}x{K} workspace")
