"""Brute-force check of the oracle on tiny inputs (CPU only).

An independent model of each path, written with exact rationals: every fp32
operation is rn32(exact result) (tests/exact_f32.py) and every rounding to the
e2m1 / e4m3 grids is an enumeration of all candidates.  It shares nothing with
the oracle except the RNG fields (pinned separately) and the input bytes, so a
wrong index, a transposed operand, a dropped term or numpy promotion slip in
the oracle's vectorised code fails here.  Inputs are finite; special values
are pinned in test_oracle_pins.py.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.nvfp4 import unpack_codes
from tests.exact_f32 import E2M1, E4M3, FLT_MAX, exact, nearest_even, rn32, to_f32

F32 = np.float32


def _inputs(seed, M, K, bf16=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-9, 9, (M, K // 16))).repeat(16, axis=1)
    x = x.astype(F32)
    x[0, :16] = 0.0                                   # an all-zero block
    x[-1, -16:] = np.float32(0.75) * x[-1, -16:].max()  # near-ties
    x[1 % M, 3] = -0.0
    if bf16:
        import workloads
        return workloads.bf16_bits(x)
    return x


def _elems(x):
    return oracle.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def _fmin(a, b):
    return a if a < b else b


def _rho(s, S_dec):
    den = rn32(s * S_dec)
    if den == 0:
        return FLT_MAX
    return _fmin(rn32(1 / den), FLT_MAX)


def _code(x: Fraction, neg: bool, rho, u16=None):
    v = rn32(abs(x) * rho)
    if v >= 6:
        idx = 7
    elif u16 is None:
        idx = nearest_even(v, E2M1)
    else:
        lo = max(i for i, g in enumerate(E2M1) if g <= v)
        f = (v - E2M1[lo]) / (E2M1[lo + 1] - E2M1[lo])
        f22 = Fraction(math.floor(f * 2 ** 22), 2 ** 22)  # fraction to 22 bits (the SR reading)
        idx = lo + (1 if Fraction(int(u16), 65536) < f22 else 0)
    return (8 if neg else 0) | idx, (-E2M1[idx] if neg else E2M1[idx])


def _model_standard(x32, global_amax=None, u16=None, residual=None):
    """Page-1 path (no global scale) or standard path (global, bound 448) on
    1x16 blocks.  Returns codes, scale bytes, x_hat (fp32), new residual."""
    M, K = x32.shape
    codes = np.zeros((M, K), np.uint8)
    sb = np.zeros((M, K // 16), np.uint8)
    xhat = np.zeros((M, K), F32)
    if global_amax is None:
        S_dec, mult = Fraction(1), None
    else:
        A, D = exact(global_amax), Fraction(2688)
        S_enc = _fmin(rn32(D / A), FLT_MAX) if A != 0 else FLT_MAX
        S_dec = rn32(A / D)
        mult = rn32(S_enc * rn32(Fraction(1, 6)))
    for m in range(M):
        for b in range(K // 16):
            xs = [x32[m, 16 * b + i] for i in range(16)]
            X = [exact(v) for v in xs]
            negs = [bool(np.signbit(v)) for v in xs]
            if residual is not None:
                rs = [residual[m, 16 * b + i] for i in range(16)]
                X = [rn32(X[i] + exact(rs[i])) for i in range(16)]
                # IEEE sign of a sum: an exact zero is -0 only for (-0) + (-0)
                negs = [X[i] < 0 or (X[i] == 0 and negs[i] and bool(np.signbit(rs[i])))
                        for i in range(16)]
            a = max(abs(v) for v in X)
            sigma = rn32(a / 6) if mult is None else rn32(a * mult)
            sigma = _fmin(sigma, Fraction(448))
            k = nearest_even(sigma, E4M3)
            s = E4M3[k]
            sb[m, b] = k
            rho = _rho(s, S_dec)
            for i in range(16):
                u = None if u16 is None else u16[m, 16 * b + i]
                c, val = _code(X[i], negs[i], rho, u)
                codes[m, 16 * b + i] = c
                xh = rn32(rn32(val * s) * S_dec)
                xhat[m, 16 * b + i] = to_f32(xh) if not (val == 0 and c & 8) else F32(-0.0)
                if residual is not None:
                    residual[m, 16 * b + i] = to_f32(rn32(X[i] - xh))
    return codes, sb, xhat


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("stochastic", [False, True])
def test_quantize_and_qdq_match_exact_model(seed, bf16, stochastic):
    M, K = 3, 48
    x = _inputs(seed, M, K, bf16)
    x32 = _elems(x)
    u16 = oracle.sr_u16(np.arange(M * K).reshape(M, K), 5, seed) if stochastic else None
    codes, sb, xhat = _model_standard(x32, u16=u16)
    packed, scales = oracle.quantize(x, stochastic=stochastic, seed=5, step=seed)
    assert np.array_equal(scales, sb)
    assert np.array_equal(unpack_codes(packed), codes)
    out = oracle.dequantize(packed, scales, M, K, out="f32")
    assert np.array_equal(out, xhat)
    # error feedback: residual in, x' = x + r, r <- x' - x_hat
    r0 = (np.random.default_rng(seed + 50).standard_normal((M, K)) * 1e-2).astype(F32)
    r_model = r0.copy()
    codes_e, sb_e, _ = _model_standard(x32, u16=u16, residual=r_model)
    r_or = r0.copy()
    _, packed_e, scales_e = oracle.qdq(x, stochastic=stochastic, residual=r_or, seed=5, step=seed)
    assert np.array_equal(scales_e, sb_e)
    assert np.array_equal(unpack_codes(packed_e), codes_e)
    assert np.array_equal(r_or.view(np.uint32), r_model.view(np.uint32))


@pytest.mark.parametrize("seed", range(3))
def test_standard_global_scale_matches_exact_model(seed):
    M, K = 2, 64
    x = _inputs(seed + 10, M, K)
    A = oracle.amax(x)
    codes, sb, xhat = _model_standard(x, global_amax=A)
    packed, scales = oracle.quantize(x, global_amax=A)
    assert np.array_equal(scales, sb)
    assert np.array_equal(unpack_codes(packed), codes)
    out = oracle.dequantize(packed, scales, M, K, global_amax=A, scale_mode="tensor", out="f32")
    assert np.array_equal(out, xhat)


def _model_4over6(x32, A_rows, err_mode, bound, block):
    """Four-over-six by enumeration; A_rows: one exact amax per row."""
    M, K = x32.shape
    D = Fraction(6 * int(bound))
    codes = np.zeros((M, K), np.uint8)
    tiles = block == "16x16"
    sb = np.zeros((M // 16, K // 16) if tiles else (M, K // 16), np.uint8)

    def groups():
        if tiles:
            for ti in range(M // 16):
                for tj in range(K // 16):
                    yield (ti, tj), [(16 * ti + r, 16 * tj + c) for r in range(16) for c in range(16)]
        else:
            for m in range(M):
                for b in range(K // 16):
                    yield (m, b), [(m, 16 * b + i) for i in range(16)]

    for key, pos in groups():
        A = A_rows[pos[0][0]]
        S_enc = _fmin(rn32(D / A), FLT_MAX) if A != 0 else FLT_MAX
        S_dec = rn32(A / D)
        X = [exact(x32[p]) for p in pos]
        a = max(abs(v) for v in X)
        sig6 = rn32(rn32(a / 6) * S_enc)
        sig4 = rn32(sig6 * Fraction(3, 2))
        cands = []
        for sig in (sig6, sig4):
            k = nearest_even(_fmin(sig, Fraction(448)), E4M3)
            s = E4M3[k]
            rho = _rho(s, S_dec)
            cs, es = [], []
            for p, xv in zip(pos, X):
                c, val = _code(xv, bool(np.signbit(x32[p])), rho)
                cs.append(c)
                d = rn32(rn32(rn32(val * s) * A) / D)
                t = rn32(xv - d)
                es.append(abs(t) if err_mode == "mae" else rn32(t * t))
            if tiles:
                rows = []
                for r in range(16):
                    acc = es[16 * r]
                    for i in range(1, 16):
                        acc = rn32(acc + es[16 * r + i])
                    rows.append(acc)
                g = rows
                L = rn32(rn32(rn32(g[0] + g[8]) + rn32(g[4] + g[12])) + rn32(rn32(g[2] + g[10]) + rn32(g[6] + g[14])))
                R = rn32(rn32(rn32(g[1] + g[9]) + rn32(g[5] + g[13])) + rn32(rn32(g[3] + g[11]) + rn32(g[7] + g[15])))
                E = rn32(L + R)
            else:
                E = es[0]
                for e in es[1:]:
                    E = rn32(E + e)
            cands.append((k, cs, E))
        (k6, c6, E6), (k4, c4, E4) = cands
        k, cs = (k4, c4) if E4 < E6 else (k6, c6)
        sb[key] = k
        for p, c in zip(pos, cs):
            codes[p] = c
    return codes, sb


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("err_mode", ["mae", "mse"])
@pytest.mark.parametrize("bound", [256, 448])
@pytest.mark.parametrize("row", [False, True])
def test_four_over_six_1x16_matches_exact_model(seed, err_mode, bound, row):
    M, K = 3, 48
    x = _inputs(seed + 20, M, K, bf16=(seed % 2 == 1))
    x32 = _elems(x)
    A = oracle.amax(x, mode="row") if row else oracle.amax(x)
    A_rows = [exact(A[m]) for m in range(M)] if row else [exact(A)] * M
    codes, sb = _model_4over6(x32, A_rows, err_mode, bound, "1x16")
    packed, scales = oracle.quantize_4over6(x, A, err_mode=err_mode, bound=bound)
    assert np.array_equal(scales, sb)
    assert np.array_equal(unpack_codes(packed), codes)


@pytest.mark.parametrize("err_mode", ["mae", "mse"])
def test_four_over_six_16x16_matches_exact_model(err_mode):
    x = _inputs(31, 32, 64)
    A = oracle.amax(x)
    codes, sb = _model_4over6(x, [exact(A)] * 32, err_mode, 256, "16x16")
    packed, scales = oracle.quantize_4over6(x, A, err_mode=err_mode, bound=256, block="16x16")
    assert np.array_equal(scales, sb)
    assert np.array_equal(unpack_codes(packed), codes)


@pytest.mark.parametrize("stochastic", [False, True])
def test_2d_matches_exact_model(stochastic):
    M, K = 32, 32
    x = _inputs(41, M, K, bf16=True)
    x32 = _elems(x)
    A = oracle.amax(x)
    Aq, D = exact(A), Fraction(2688)
    S_enc = _fmin(rn32(D / Aq), FLT_MAX)
    S_dec = rn32(Aq / D)
    mult = rn32(S_enc * rn32(Fraction(1, 6)))
    u16 = oracle.sr_u16(np.arange(M * K).reshape(M, K), 2, 9) if stochastic else None
    codes = np.zeros((M, K), np.uint8)
    sb = np.zeros((M // 16, K // 16), np.uint8)
    for ti in range(M // 16):
        for tj in range(K // 16):
            blk = [(16 * ti + r, 16 * tj + c) for r in range(16) for c in range(16)]
            a = max(abs(exact(x32[p])) for p in blk)
            k = nearest_even(_fmin(rn32(a * mult), Fraction(448)), E4M3)
            sb[ti, tj] = k
            rho = _rho(E4M3[k], S_dec)
            for p in blk:
                codes[p] = _code(exact(x32[p]), bool(np.signbit(x32[p])), rho,
                                 None if u16 is None else u16[p])[0]
    r, c, s = oracle.quantize_2d(x, stochastic=stochastic, seed=2, step=9, global_amax=A)
    assert np.array_equal(s, sb)
    assert np.array_equal(unpack_codes(r), codes)
    assert np.array_equal(unpack_codes(c), codes.T)


def test_tile_error_tree_order():
    # Four-over-six pull request, CuTe DSL kernel Design: the 16 row errors of
    # a 16x16 tile are combined by one fixed width-16 tree.  Mixed magnitudes
    # make every association give a different fp32 result, so only that tree
    # (evaluated here with exact rationals) matches, and every term counts.
    from oracle.nvfp4 import _tree16
    rng = np.random.default_rng(0)
    e = (rng.uniform(1, 2, (400, 16)) * 2.0 ** rng.integers(-30, 30, (400, 16))).astype(F32)
    got = _tree16(e)
    for row, g_or in zip(e, got):
        g = [exact(v) for v in row]
        L = rn32(rn32(rn32(g[0] + g[8]) + rn32(g[4] + g[12])) + rn32(rn32(g[2] + g[10]) + rn32(g[6] + g[14])))
        R = rn32(rn32(rn32(g[1] + g[9]) + rn32(g[5] + g[13])) + rn32(rn32(g[3] + g[11]) + rn32(g[7] + g[15])))
        assert to_f32(rn32(L + R)) == g_or
    # all sixteen terms enter: distinct powers of two sum exactly
    p = (2.0 ** np.arange(16)).astype(F32)[None, :]
    assert _tree16(p)[0] == F32(2 ** 16 - 1)
