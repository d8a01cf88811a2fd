"""Seeded synthetic inputs for the NVFP4 quantization workloads.

This module only draws random numbers and casts them; it holds none of the
quantization arithmetic.  Both the CPU oracle (through the tests) and the HIP
path (through the tests and the benchmark) are fed from here, so the two sides
see the same bytes.

Every generator is `numpy.random.default_rng` (PCG64) with a fixed seed.  bf16
tensors are returned as `uint16` bit patterns, rounded from float32 with
round-to-nearest-even by torch's CPU cast (a library routine, kept apart from
the oracle's own bf16 conversion).

Workloads (shapes and value distributions stand in for the pages' LLM weights,
activations and gradients, which are not available):

* small      - 256x256 fp32, N(0,1), data seed 0.
* ef_weight  - 4096x4096 stored weight, W0 = bf16(0.02 * N(0,1)) (seed 0);
               per-step gradient g_t ~ N(0,1) drawn from seed (1, t).
* act_rows   - 8192x7168 bf16 activation: z ~ N(0,1) (seed 0), one std per row
               sigma_i = 10**(4 u_i - 2) with u ~ U[0,1) (seed 1), x = bf16(sigma_i z).
* weight_2d  - 7168x18432 bf16 weight: 0.02 * N(0,1) (seed 0), entries with a
               U[0,1) draw below 0.001 (seed 1) scaled by 50.
* heavy_act  - 16384x8192 bf16 heavy-tailed activation: Student-t (df=3)
               (seed 7); elements with a U[0,1) draw below 0.01 (seed 17) scaled
               by 100; per 16-element block v ~ U[0,1) (seed 27): v < 0.02 sets
               the block to zero, 0.02 <= v < 0.03 rescales it so its absmax is
               2**-10 * (1 + v') with v' ~ U[0,1) (seed 37), below the smallest
               e4m3 block scale.  Residual: zeros, or 0.01 * N(0,1) (seed 8).
"""
from __future__ import annotations

import numpy as np

SMALL_SHAPE = (256, 256)
EF_SHAPE = (4096, 4096)
EF_STEPS = 500
EF_LR = 1e-4
ACT_ROWS_SHAPE = (8192, 7168)
WEIGHT_2D_SHAPE = (7168, 18432)
HEAVY_SHAPE = (16384, 8192)
HEAVY_SEED, HEAVY_STEP = 7, 123


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (RNE, via torch's CPU cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal(seed, shape, scale=1.0) -> np.ndarray:
    z = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        z *= np.float32(scale)
    return z


def small_input(shape=SMALL_SHAPE, seed=0) -> np.ndarray:
    """fp32 N(0,1) tensor (the 256x256 quantize/dequantize case)."""
    return normal(seed, shape)


def ef_weight0(shape=EF_SHAPE, seed=0) -> np.ndarray:
    """bf16 bits of the initial stored weight, 0.02 * N(0,1)."""
    return bf16_bits(normal(seed, shape, 0.02))


def ef_grad(step: int, shape=EF_SHAPE, rows: int | None = None) -> np.ndarray:
    """fp32 N(0,1) gradient of one step, seed (1, step).

    numpy fills arrays in C order from one stream, so `rows=r` returns exactly
    the first r rows of the full-size draw at a fraction of the cost.
    """
    m = shape[0] if rows is None else rows
    rng = np.random.default_rng([1, step])
    return rng.standard_normal((m, shape[1]), dtype=np.float32)


def act_rows_input(shape=ACT_ROWS_SHAPE, seed_z=0, seed_u=1) -> np.ndarray:
    """bf16 bits: N(0,1) with a log-uniform per-row std in [1e-2, 1e2]."""
    z = normal(seed_z, shape)
    u = np.random.default_rng(seed_u).random(shape[0])
    sig = (10.0 ** (4.0 * u - 2.0)).astype(np.float32)
    z *= sig[:, None]
    return bf16_bits(z)


def weight_2d_input(shape=WEIGHT_2D_SHAPE, seed=0, seed_mask=1, frac=0.001, boost=50.0) -> np.ndarray:
    """bf16 bits: 0.02 * N(0,1) with a sparse set of x50 entries."""
    w = normal(seed, shape, 0.02)
    mask = np.random.default_rng(seed_mask).random(shape, dtype=np.float32) < np.float32(frac)
    w[mask] *= np.float32(boost)
    return bf16_bits(w)


def heavy_input(shape=HEAVY_SHAPE, seed=7, seed_mask=17, seed_block=27, seed_tiny=37) -> np.ndarray:
    """bf16 bits: Student-t(3) with outliers, zero blocks and sub-scale blocks."""
    m, k = shape
    x = np.random.default_rng(seed).standard_t(3, size=shape).astype(np.float32)
    out = np.random.default_rng(seed_mask).random(shape, dtype=np.float32) < np.float32(0.01)
    x[out] *= np.float32(100.0)
    xb = x.reshape(m, k // 16, 16)
    v = np.random.default_rng(seed_block).random((m, k // 16))
    xb[v < 0.02] = 0.0
    tiny = (v >= 0.02) & (v < 0.03)
    vt = np.random.default_rng(seed_tiny).random((m, k // 16))
    target = (2.0 ** -10) * (1.0 + vt)
    amax = np.abs(xb).max(axis=2).astype(np.float64)
    amax[amax == 0] = 1.0
    fac = (target / amax).astype(np.float32)
    xb[tiny] *= fac[tiny][:, None]
    return bf16_bits(x)


def heavy_residual(shape=HEAVY_SHAPE, seed=8) -> np.ndarray:
    """fp32 starting residual 0.01 * N(0,1)."""
    return normal(seed, shape, 0.01)
