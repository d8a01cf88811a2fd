"""Pins for the oracle's extension paths (CPU only): the truncation-free 2D
scale, four-over-six on 16x16 tiles with row + column outputs, and the fused
rowwise + columnwise 1x16 quantization."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.nvfp4 import code_values, pack_codes, unpack_codes
from tests.exact_f32 import E4M3, exact

F32 = np.float32


def test_e4m3_round_up_is_the_smallest_value_not_below():
    rng = np.random.default_rng(0)
    sig = np.concatenate([(2.0 ** rng.uniform(-14, 9, 3000)).astype(F32), oracle.E4M3_VALUES,
                          np.nextafter(oracle.E4M3_VALUES, F32(np.inf)), np.array([0, 500, 1e30], F32)])
    codes = oracle.e4m3_encode_up(sig)
    for s, c in zip(sig, codes):
        c = int(c)
        if exact(s) > E4M3[-1]:
            assert c == 0x7E
            continue
        assert E4M3[c] >= exact(s)
        assert c == 0 or E4M3[c - 1] < exact(s)
    # exact e4m3 values are their own round-up; otherwise one above nearest or equal
    assert np.array_equal(oracle.e4m3_encode_up(oracle.E4M3_VALUES), np.arange(127, dtype=np.uint8))
    rne = oracle.e4m3_encode(np.fmin(sig, 448))
    assert np.all((codes == rne) | (codes == rne + 1))


@pytest.mark.parametrize("global_scale", [False, True])
def test_truncation_free_2d_never_saturates(global_scale):
    # With the scale rounded up, s >= a / 6 and every |x| * rho <= 6 (up to
    # the rounding of rho), so SR never clips: each dequantized value lies on
    # one of the two grid points around x.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 64)) * np.exp(rng.uniform(-4, 4, (64, 64)))).astype(F32)
    A = oracle.amax(x) if global_scale else None
    r, c, s = oracle.quantize_2d(x, stochastic=True, seed=1, step=2, global_amax=A, truncation_free=True)
    r0, _, s0 = oracle.quantize_2d(x, stochastic=True, seed=1, step=2, global_amax=A)
    assert np.all((s == s0) | (s == s0 + 1))
    S_dec = np.float32(1.0) if A is None else oracle.nvfp4.global_scales(A, 448.0)[1]
    sv = np.repeat(np.repeat(oracle.E4M3_VALUES[s], 16, 0), 16, 1).astype(np.float64) * float(S_dec)
    q = np.abs(code_values(unpack_codes(r)).astype(np.float64))
    v = np.abs(x.astype(np.float64)) / sv
    lo = oracle.E2M1_GRID[np.clip(np.searchsorted(oracle.E2M1_GRID, v, side="right") - 1, 0, 7)]
    assert np.all(v <= 6.0 * (1 + 2.0 ** -20))
    assert np.all((q == lo) | (q > lo))
    assert np.all(q - v < 2.0 + 1e-9)
    # the nearest-scale variant does clip on this input
    q0 = np.abs(code_values(unpack_codes(r0)).astype(np.float64))
    assert (np.abs(x).astype(np.float64) /
            (np.repeat(np.repeat(oracle.E4M3_VALUES[s0], 16, 0), 16, 1) * float(S_dec)) > 6).any()
    assert q0.max() == 6.0


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_four_over_six_2d_outputs(err):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((48, 64)) * np.exp(rng.uniform(-3, 3, (48, 1)))).astype(F32)
    A = oracle.amax(x)
    pr, pc, ts = oracle.quantize_4over6_2d(x, A, err_mode=err)
    p16, s16 = oracle.quantize_4over6(x, A, err_mode=err, block="16x16")
    assert np.array_equal(pr, p16) and np.array_equal(ts, s16)
    assert np.array_equal(pc, pack_codes(unpack_codes(pr).T))
    assert ts.shape == (3, 4) and ts.max() <= 0x7C


@pytest.mark.parametrize("four_over_six,bound", [(False, 448.0), (True, 256.0), (True, 448.0)])
def test_rowcol_swaps_under_transpose(four_over_six, bound):
    rng = np.random.default_rng(7)
    x = oracle.f32_to_bf16_bits((rng.standard_normal((32, 80)) * 3).astype(F32))
    A = oracle.amax(x)
    pr, sr, pc, sc = oracle.quantize_rowcol(x, A, four_over_six=four_over_six, bound=bound)
    xt = np.ascontiguousarray(x.T)
    prt, srt, pct, sct = oracle.quantize_rowcol(xt, A, four_over_six=four_over_six, bound=bound)
    assert np.array_equal(pr, pct) and np.array_equal(sr, sct)
    assert np.array_equal(pc, prt) and np.array_equal(sc, srt)
    if not four_over_six:
        p, s = oracle.quantize(x, global_amax=A)
        assert np.array_equal(p, pr) and np.array_equal(s, sr)
