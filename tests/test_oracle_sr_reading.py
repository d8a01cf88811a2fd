"""Pins of the oracle's stochastic-rounding reading against the fp4-train
card, Method: between two neighbouring e2m1 grid points lo <= v < hi, the
value goes up to hi with probability equal to its fractional distance
f = (v - lo) / (hi - lo).

The card fixes neither the draw's resolution nor the comparison.  The oracle
draws u = u16 * 2^-16 and rounds up iff u < f22, with f22 = f truncated to 22
fractional bits.  Nothing here retypes that rule.  Instead, for each tested v,
the test counts how many of the 65,536 possible draws the oracle's encoder
rounds up.  That count is found by bisection over u16, since the encoder is
monotone in the draw.  The resulting probability P(up) is then compared with
f, which the test computes in float64 from the grid.  The card's requirement,
up to the 16-bit draw, is |P(up) - f| < 2^-16 in every binade below 6.
Subnormal fp32 values are included.  A mean test at 0.7 and at 2.3 (unit
scale) checks the same thing through the quantize and dequantize entry
points, using the oracle's own counter-based draws.
"""
import numpy as np
import pytest

import oracle

F32 = np.float32
GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _bracket(v):
    v64 = v.astype(np.float64)
    lo = np.clip(np.searchsorted(GRID, v64, side="right") - 1, 0, 6)
    return lo, GRID[lo], GRID[lo + 1]


def _p_up(v):
    """Number of u16 in [0, 65536) for which the oracle rounds v up, by
    bisection on the draw (the encoder is monotone in u16)."""
    lo_idx, _, _ = _bracket(v)
    lo = np.zeros(v.shape, np.int64)          # every u < lo rounds up
    hi = np.full(v.shape, 65536, np.int64)    # every u >= hi stays down
    for _ in range(17):
        mid = (lo + hi) // 2
        probe = np.minimum(mid, 65535)
        up = oracle.e2m1_sr_index(v, probe) > lo_idx
        go = (mid < 65536) & up
        lo = np.where(go, mid + 1, lo)
        hi = np.where(go, hi, mid)
    return lo


def _binade_values(e_field, rng, n):
    """Float32 values with biased exponent e_field (0 = subnormal): random
    mantissas plus mantissas whose low bits are all zero, all one, or a
    single set bit (fractions that end exactly at, or just past, the 22nd
    fractional bit)."""
    special = [0, 1, 2, 3, (1 << 23) - 1, (1 << 22), (1 << 22) - 1, 0x155555, 0x2AAAAA]
    special += [1 << k for k in range(23)] + [(1 << 23) - (1 << k) for k in range(23)]
    mant = np.concatenate([rng.integers(0, 1 << 23, n, dtype=np.uint32), np.array(special, np.uint32)])
    v = ((np.uint32(e_field) << np.uint32(23)) | mant).view(np.float32)
    return v[(v < F32(6.0)) & (v > 0)]


def test_sr_probability_is_the_fractional_distance_in_every_binade():
    rng = np.random.default_rng(0)
    worst = 0.0
    for e in range(0, 130):  # subnormals, then every binade from 2^-126 up to [4, 8)
        v = _binade_values(e, rng, 2048)
        cnt = _p_up(v)
        _, glo, ghi = _bracket(v)
        f = (v.astype(np.float64) - glo) / (ghi - glo)  # exact in float64
        P = cnt / 65536.0
        d = P - f
        assert np.all(d < 2.0 ** -16), (e, v[np.argmax(d)])
        assert np.all(d > -(2.0 ** -22)), (e, v[np.argmin(d)])
        # on-grid values never move; a positive fraction always has some chance
        # of moving unless it is below 2^-22 (the truncation step)
        assert np.all(cnt[f == 0] == 0)
        assert np.all(cnt[f >= 2.0 ** -22] > 0)
        if e >= 127:  # v >= 1: every f has at most 22 fractional bits
            assert np.array_equal(cnt, np.ceil(f * 65536.0).astype(np.int64)), e
        worst = max(worst, float(np.abs(d).max()))
    assert worst < 2.0 ** -16


def test_sr_expected_value_is_unbiased_to_the_draw_resolution():
    # E[q] = lo + (hi - lo) P(up); its distance from v is (hi - lo) |P - f|.
    rng = np.random.default_rng(1)
    v = rng.uniform(0, 6, 20000).astype(F32)
    cnt = _p_up(v)
    _, glo, ghi = _bracket(v)
    Eq = glo + (ghi - glo) * cnt / 65536.0
    assert np.all(np.abs(Eq - v.astype(np.float64)) < (ghi - glo) * 2.0 ** -16)


def _unit_block_mean(value, blocks, steps):
    """Mean dequantized value of `value` in unit-scale blocks [6, value x 15]
    over `blocks` blocks and the given SR steps (quantize + dequantize)."""
    x = np.full((blocks, 16), F32(value), F32)
    x[:, 0] = 6.0
    x = x.reshape(-1, 256)
    M, K = x.shape
    acc, n = 0.0, 0
    for step in steps:
        p, s = oracle.quantize(x, stochastic=True, seed=11, step=step)
        assert np.all(s == 0x38)  # block amax 6 -> scale 1.0 (e4m3 0x38)
        d = oracle.dequantize(p, s, M, K, out="f32").reshape(-1, 16)[:, 1:]
        acc += float(d.astype(np.float64).sum())
        n += d.size
    return acc / n, n


@pytest.mark.parametrize("value", [0.7, 2.3])
def test_sr_mean_at_unit_scale(value):
    v = F32(value)
    mean, n = _unit_block_mean(value, 1 << 14, range(4))
    _, glo, ghi = _bracket(np.array([v]))
    f = (float(v) - glo[0]) / (ghi[0] - glo[0])
    sd = (ghi[0] - glo[0]) * np.sqrt(f * (1 - f) / n)
    assert abs(mean - float(v)) < 3 * sd + (ghi[0] - glo[0]) * 2.0 ** -16
    assert f"{mean:.3f}" == f"{value:.3f}"
