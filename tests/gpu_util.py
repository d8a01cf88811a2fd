"""Helpers for the GPU parity tests: move seeded numpy inputs to the device
and bring results back as numpy bit patterns."""
from __future__ import annotations

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    raise TypeError(x.dtype)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """View for bitwise comparison (float32 -> uint32)."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_bitwise(got, want, what=""):
    g, w = bits(np.asarray(got)), bits(np.asarray(want))
    assert g.shape == w.shape, (what, g.shape, w.shape)
    if not np.array_equal(g, w):
        bad = np.argwhere(g != w)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {g[i]!r} want {w[i]!r}")


def wide_input(seed, M, K, bf16=False, lo=-12.0, hi=12.0):
    """N(0,1) values with a log-uniform scale per 16-element block (e**lo ..
    e**hi), an all-zero block and a -0; bf16 bits if requested."""
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.uniform(lo, hi, (M, max(K // 16, 1)))).repeat(16, axis=1)[:, :K]
    x = (rng.standard_normal((M, K)) * scale).astype(np.float32)
    if M * K >= 32:
        x.reshape(-1)[:16] = 0.0
        x.reshape(-1)[17] = -0.0
    if bf16:
        import workloads
        return workloads.bf16_bits(x)
    return x
