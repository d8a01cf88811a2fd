"""Dense checks of the hardware-assisted encode paths against the oracle.

The round-to-nearest kernels take element codes from the gfx950 fp32 -> e2m1
conversion and scale bytes from the fp32 -> e4m3 conversion.  Here the
ordinary quantize entry point is driven so that those conversions see dense
sweeps of their inputs, and every code and scale byte is compared with the
CPU oracle:

* element codes: blocks [6, v_1 .. v_15] have amax 6, scale 1.0 and encode
  reciprocal 1, so each v is rounded as it stands; the v sweep every float32
  in [0, 8) whose low 6 mantissa bits are zero, +-2^12 ulps around every
  rounding midpoint, and both signs;
* scale bytes: one block per amax value, over every positive finite bf16
  value up to 2688 (sigma = a / 6 up to 448) and 2^20 float32 values;
* stochastic rounding (the hardware stochastic-rounding conversion with one
  16-bit draw per element): unit-scale blocks holding values across every
  binade below 6 (fp32 subnormals included), values just around every grid
  point, and values whose fraction ends below the 22nd bit, each under
  several (seed, step) streams, so that many draws land on the truncation
  boundary; codes, residuals and dequantized values are compared.
"""
import numpy as np
import pytest
import torch

import oracle
import fp4_block_quantization_nvfp4_amd as nv
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _unit_scale_blocks(v):
    n = (len(v) + 14) // 15
    vv = np.zeros(n * 15, np.float32)
    vv[: len(v)] = v
    x = np.empty((n, 16), np.float32)
    x[:, 0] = 6.0
    x[:, 1:] = vv.reshape(n, 15)
    return x.reshape(-1, 64) if n % 4 == 0 else x


def test_e2m1_conversion_dense_sweep():
    grid = np.arange(0, 0x41000000, 64, dtype=np.uint32).view(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-4096, 4097)[None, :]).reshape(-1).astype(np.uint32)
    v = np.concatenate([grid, near.view(np.float32)])
    v = np.concatenate([v, -v, np.array([7.0, 1e30, -1e30, np.inf, -np.inf, 0.0, -0.0], np.float32)])
    for chunk in np.array_split(v, 4):
        x = _unit_scale_blocks(chunk)
        M, K = x.shape
        wp, ws = oracle.quantize(x)
        p, s = nv.quantize(to_dev(x))
        assert_bitwise(to_np(s), ws, "scales")
        assert_bitwise(to_np(p), wp, "codes")


def test_e4m3_scale_dense_sweep():
    b = np.arange(1, 0x7F80, dtype=np.uint32)
    a_bf16 = (b << 16).view(np.float32)
    a_bf16 = a_bf16[a_bf16 <= 2688.0]
    rng = np.random.default_rng(0)
    a_f32 = (2.0 ** rng.uniform(-20, np.log2(3000.0), 1 << 20)).astype(np.float32)
    for a in (a_bf16, a_f32):
        x = np.zeros((len(a), 16), np.float32)
        x[:, 0] = a
        x[:, 1] = -a * np.float32(0.5)
        for dt in ("f32", "bf16"):
            xin = x if dt == "f32" else oracle.f32_to_bf16_bits(x)
            wp, ws = oracle.quantize(xin)
            p, s = nv.quantize(to_dev(xin))
            assert_bitwise(to_np(s), ws, f"scales {dt}")
            assert_bitwise(to_np(p), wp, f"codes {dt}")


def test_stochastic_rounding_dense_sweep():
    rng = np.random.default_rng(4)
    n = 1 << 19
    ex = rng.integers(0, 130, n).astype(np.uint32)           # binades 2^-126 .. 2^2, and subnormals
    v = ((ex << 23) | rng.integers(0, 1 << 23, n, dtype=np.uint32)).view(np.float32)
    v = v[v < 6.0]
    grid = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0], np.float32).view(np.uint32)
    near = (grid[:, None].astype(np.int64) + np.arange(-512, 513)[None, :]).reshape(-1).astype(np.uint32)
    v = np.concatenate([v, near.view(np.float32), np.array([0.0, 6.0, 7.0, np.inf], np.float32)])
    v = np.where(rng.random(v.shape) < 0.5, -v, v).astype(np.float32)
    x = _unit_scale_blocks(v)
    xd = to_dev(x)
    for seed, step in ((0, 0), (7, 123), (0xDEADBEEF, 0xFFFFFFFF)):
        wp, ws = oracle.quantize(x, stochastic=True, seed=seed, step=step)
        p, s = nv.quantize(xd, stochastic=True, seed=seed, step=step)
        assert_bitwise(to_np(s), ws, f"scales seed={seed}")
        assert_bitwise(to_np(p), wp, f"codes seed={seed}")
        r = np.zeros_like(x)
        wo = oracle.qdq(x, stochastic=True, residual=r, seed=seed, step=step, out="f32")[0]
        rd = torch.zeros_like(xd)
        got = nv.qdq(xd, stochastic=True, residual=rd, seed=seed, step=step, out_dtype=torch.float32)
        assert_bitwise(to_np(got), wo, f"qdq seed={seed}")
        assert_bitwise(to_np(rd), r, f"residual seed={seed}")
    x2 = np.ascontiguousarray(x[: x.shape[0] // 16 * 16])
    wr, wc, wt = oracle.quantize_2d(x2, stochastic=True, seed=3, step=4)
    r2, c2, t2 = nv.quantize_2d(to_dev(x2), stochastic=True, seed=3, step=4)
    assert_bitwise(to_np(t2), wt, "2d tile scales")
    assert_bitwise(to_np(r2), wr, "2d rowwise")
    assert_bitwise(to_np(c2), wc, "2d columnwise")


@pytest.mark.parametrize("seed,step", [(0, 0), (7, 123), (0xDEADBEEF, 5)])
def test_stochastic_rounding_on_each_elements_draw_boundary(seed, step):
    """Unit-scale blocks [6, v_1 .. v_15] where every v_i is placed from
    element i's own draw u_i (the counter-based stream of the fp4-train
    card, Method): its fractional distance in a grid interval is exactly
    u_i * 2^-16 (stays down), or that plus 2^-24, 2^-23 (below the 22-bit
    truncation: stays down under the library's reading) or 2^-22 (goes up).
    Intervals cycle over all seven, so every binade of the scaled value from
    2^-17 to 6 sees boundary cases; quantize, qdq + residual and the 2D pass
    are compared with the oracle."""
    n_blocks = 1 << 14
    M, K = n_blocks // 4, 64
    idx = np.arange(M * K, dtype=np.int64).reshape(M, K)
    u = oracle.sr_u16(idx, seed, step).astype(np.float64)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    k = (idx // 16 + idx) % 7                           # interval [grid[k], grid[k+1])
    delta = np.array([0.0, 2.0 ** -24, 2.0 ** -23, 2.0 ** -22])[(idx // 7) % 4]
    v = grid[k] + (u / 65536.0 + delta) * (grid[k + 1] - grid[k])
    # an offset finer than the fp32 spacing of its interval becomes 2^-22
    fine = v.astype(np.float32).astype(np.float64) != v
    v = np.where(fine, grid[k] + (u / 65536.0 + 2.0 ** -22) * (grid[k + 1] - grid[k]), v)
    x = v.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), v)   # every v is exact in fp32
    x = np.where((idx // 3) % 2 == 1, -x, x).astype(np.float32)
    x[:, ::16] = 6.0                                   # block amax 6: scale 1, rho 1
    xd = to_dev(x)
    wp, ws = oracle.quantize(x, stochastic=True, seed=seed, step=step)
    p, s = nv.quantize(xd, stochastic=True, seed=seed, step=step)
    assert np.all(ws == 0x38)
    assert_bitwise(to_np(s), ws, "scales")
    assert_bitwise(to_np(p), wp, "codes")
    r = np.zeros_like(x)
    wo = oracle.qdq(x, stochastic=True, residual=r, seed=seed, step=step, out="f32")[0]
    rd = torch.zeros_like(xd)
    got = nv.qdq(xd, stochastic=True, residual=rd, seed=seed, step=step, out_dtype=torch.float32)
    assert_bitwise(to_np(got), wo, "qdq")
    assert_bitwise(to_np(rd), r, "residual")
    wr, wc, wt = oracle.quantize_2d(x, stochastic=True, seed=seed, step=step)
    r2, c2, t2 = nv.quantize_2d(xd, stochastic=True, seed=seed, step=step)
    assert_bitwise(to_np(t2), wt, "2d tile scales")
    assert_bitwise(to_np(r2), wr, "2d rowwise")
    assert_bitwise(to_np(c2), wc, "2d columnwise")
