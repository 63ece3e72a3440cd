"""Helpers for the GPU tests: host <-> device copies of bit patterns."""
import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible gfx950 GPU")
    return torch.device("cuda:0")


def to_dev_u16(a: np.ndarray, dev=None) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a torch bf16 tensor on the GPU."""
    a = np.ascontiguousarray(a, np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev or device())


def to_dev(a: np.ndarray, dev=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev or device())


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def first_mismatch(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return None
    i = tuple(idx[0])
    return f"{idx.shape[0]} mismatches; first at {i}: got {a[i]!r}, want {b[i]!r}"
