"""Exact rational model of IEEE binary32 round-to-nearest-even, for
brute-force checks of the oracle on tiny inputs.

fl(a op b) is computed as rn32(exact(a) op exact(b)) with Python Fractions,
so nothing here depends on numpy's float32 arithmetic.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

FLT_MAX = Fraction((2 ** 24 - 1) * 2 ** 104)
INF = float("inf")
_OVER = Fraction(2 ** 128 - 2 ** 103)  # the RNE overflow threshold


def exact(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def rn32(q):
    """Nearest binary32 value to the rational q, ties to even; returns a
    Fraction, or +-inf (float) on overflow."""
    if isinstance(q, float):
        return q
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    if a >= _OVER:
        return sign * INF
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return sign * (k * quantum)


def to_f32(q) -> np.float32:
    return np.float32(float(q))


def nearest_even(v: Fraction, table):
    """Index of the nearest table value (exact Fractions), ties to the even
    index, by enumeration; v above the table saturates to the last index."""
    if v >= table[-1]:
        return len(table) - 1
    best = None
    for i, t in enumerate(table):
        d = abs(v - t)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


E2M1 = [Fraction(x) for x in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def e4m3_table():
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        vals.append(Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


E4M3 = e4m3_table()
