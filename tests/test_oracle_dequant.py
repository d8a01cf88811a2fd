"""Exact-rational pins of every branch of oracle.dequantize (fp4-train, API:
dequantize(packed, scale, M, K) -> bf16; four-over-six pull request, What:
a scalar global_amax is per-tensor scaling, a (rows,) vector the row-wise
variant; 16x16 tiles share one scale per tile).

The model decodes each nibble by hand (even element in the low nibble,
code = sign << 3 | magnitude index into the e2m1 grid), looks up the scale
byte of the element's block (1x16: [m, k // 16]; tile16: [m // 16, k // 16])
and the second-level S_dec = fl(A / (6 * bound)) of its tensor or row, and
forms fl(fl(val * s) * S_dec) with exact rationals, then rounds to bf16 by
round-to-nearest-even on the rational (8 significant bits).  Nothing is
shared with the oracle's vectorised code.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact_f32 import E2M1, E4M3, exact, rn32, to_f32

F32 = np.float32


def rn_bf16(q):
    """Nearest bfloat16 to a rational (8 significant bits, float32 exponent
    range, subnormal quantum 2^-133), ties to even; +-inf on overflow."""
    if isinstance(q, float) or q == 0:
        return q
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 7)
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    r = k * quantum
    if r >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * r


def _bf16_bits(q, neg_zero):
    if q == 0:
        return 0x8000 if neg_zero else 0
    f = np.array([float(q)], np.float32)  # exact: q is a bf16 value
    return int(f.view(np.uint32)[0] >> 16)


def _model(packed, scales, M, K, tile16, A, bound):
    """x_hat as float32 and as bf16 bits, element by element."""
    out32 = np.zeros((M, K), F32)
    out16 = np.zeros((M, K), np.uint16)
    D = Fraction(int(6 * bound))
    for m in range(M):
        if A is None:
            S_dec = Fraction(1)
        else:
            Am = A[m] if np.ndim(A) == 1 else A
            S_dec = rn32(exact(Am) / D)
        for k in range(K):
            byte = int(packed[m, k // 2])
            code = (byte >> 4) if k % 2 else (byte & 0xF)
            neg = bool(code & 8)
            val = E2M1[code & 7] * (-1 if neg else 1)
            sb = int(scales[m // 16, k // 16]) if tile16 else int(scales[m, k // 16])
            s = E4M3[sb]
            xh = rn32(rn32(val * s) * S_dec)
            nz = xh == 0 and neg
            out32[m, k] = F32(-0.0) if nz else to_f32(xh)
            out16[m, k] = _bf16_bits(rn_bf16(xh), nz)
    return out32, out16


def _inputs(seed, M, K, tile16):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    sshape = (M // 16, K // 16) if tile16 else (M, K // 16)
    scales = rng.integers(0, 127, sshape, dtype=np.uint8)
    scales.reshape(-1)[:3] = [0, 1, 0x7E]  # zero, smallest subnormal, largest scale
    return packed, scales


# Row-wise scaling is 1x16 only, and the bound only matters with a global
# scale: those combinations are left out.
_CASES = [(t, m, b) for t in (False, True) for m in ("none", "tensor", "row") for b in (256.0, 448.0)
          if not (t and m == "row") and not (m == "none" and b == 256.0)]


@pytest.mark.parametrize("tile16,mode,bound", _CASES,
                         ids=[f"{'tile16' if t else '1x16'}-{m}-{int(b)}" for t, m, b in _CASES])
def test_dequantize_matches_exact_model(tile16, mode, bound):
    M, K = 32, 48
    packed, scales = _inputs(int(bound) + (7 if tile16 else 0), M, K, tile16)
    rng = np.random.default_rng(3)
    A = None
    if mode == "tensor":
        A = F32(rng.uniform(0.01, 100.0))
    elif mode == "row":
        A = np.exp(rng.uniform(-12, 12, M)).astype(F32)
        A[0] = 0.0                     # an all-zero row: S_dec = 0
        A[1] = F32(3e38)               # a huge amax: products overflow to inf
    want32, want16 = _model(packed, scales, M, K, tile16, A, bound)
    kw = dict(tile16=tile16, scale_mode=mode, bound=bound)
    if mode != "none":
        kw["global_amax"] = A
    got32 = oracle.dequantize(packed, scales, M, K, out="f32", **kw)
    got16 = oracle.dequantize(packed, scales, M, K, out="bf16", **kw)
    assert np.array_equal(got32.view(np.uint32), want32.view(np.uint32))
    assert np.array_equal(got16, want16)


def test_row_dequantize_inverts_row_scaled_four_over_six():
    # The dequantized row-scaled four-over-six codes are the candidates'
    # d = ((val * s) * A) / D up to the placement of the rounding: x_hat =
    # (val * s) * fl(A / D) lies within 1.5 ulp of it and keeps its sign.
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((8, 64)) * np.exp(rng.uniform(-6, 6, (8, 1)))).astype(F32)
    A = oracle.amax(x, mode="row")
    p, s = oracle.quantize_4over6(x, A, err_mode="mae", bound=256.0)
    xh = oracle.dequantize(p, s, 8, 64, scale_mode="row", global_amax=A, bound=256.0, out="f32")
    codes = np.empty((8, 64), np.int64)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    val = np.array([float(g) for g in E2M1])[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    sv = np.array([float(E4M3[b]) for b in s.reshape(-1)]).reshape(s.shape).repeat(16, axis=1)
    d = val * sv * A.astype(np.float64)[:, None] / 1536.0
    assert np.all(np.abs(xh - d) <= 1.5 * np.spacing(np.abs(d).astype(F32)) + 1e-45)
    assert np.all(np.abs(xh.astype(np.float64) - x) <= np.abs(x) + 1e-30)
