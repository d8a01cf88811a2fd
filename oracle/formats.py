"""Element and scale formats (oracle; test infrastructure only).

* e2m1: the 4-bit element format, a sign bit and the magnitude grid
  {0, .5, 1, 1.5, 2, 3, 4, 6} ("fp4-train", Method).  Magnitude index 0..7 in
  grid order; code = sign << 3 | index.
* e4m3: the OCP E4M3FN block-scale byte, 4 exponent bits (bias 7), 3 mantissa
  bits, largest finite value 448 (four-over-six pull request, What: the bound
  argument 256*1.5 = 384 < 448).  Only the 127 finite non-negative codes
  0x00..0x7E occur as scales; their value order equals their code order.
* Rounding to either grid is to the nearest value with ties to the even
  index (round-to-nearest-even), saturating at the largest value - the
  "RTNE" of the four-over-six pull request (What) and its satfinite casts
  (CuTe DSL kernel, Design).
* bf16: float32 -> bf16 by round-to-nearest-even on the bit pattern; NaN maps
  to the canonical quiet NaN 0x7FC0 (a choice; the pages do not say).

Everything here is written from the format definitions.  It is pinned in
tests/test_oracle_formats.py against torch's float8_e4m3fn and bfloat16 casts
(library routines), exact rational brute force, and the byte values the
format fixes.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
FLT_MAX = np.float32(np.finfo(np.float32).max)

# fp4-train, Method: the e2m1 grid.
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def e4m3_decode(code) -> np.ndarray:
    """e4m3 byte (0..126) -> float32 value.

    Exponent field e = code >> 3, mantissa m = code & 7; e == 0 is subnormal
    m * 2**-9, otherwise (1 + m/8) * 2**(e - 7).
    """
    code = np.asarray(code, dtype=np.int64)
    e = code >> 3
    m = code & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return val.astype(np.float32)


# The 127 finite non-negative e4m3 values, indexed by code.
E4M3_VALUES = e4m3_decode(np.arange(127))


def _nearest_even_index(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to v (v >= 0, not NaN), ties to the
    even index, saturating at the last index for v above the table.

    The table is sorted ascending and starts at 0.  Comparisons run in
    float64, where both distances to the two neighbours are exact (the
    neighbours are within a factor 2 of v, or the lower one is 0).
    """
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    t = table.astype(np.float64)
    n = len(t)
    hi = np.searchsorted(t, v64, side="left")  # t[hi-1] < v <= t[hi]
    hi_c = np.minimum(hi, n - 1)
    lo_c = np.maximum(hi - 1, 0)
    d_lo = v64 - t[lo_c]
    d_hi = t[hi_c] - v64
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    idx = np.where(pick_hi, hi_c, lo_c)
    idx = np.where(hi >= n, n - 1, idx)
    idx = np.where(hi == 0, 0, idx)
    return idx.astype(np.int64)


def e4m3_encode(sigma) -> np.ndarray:
    """fp32 scale sigma (>= 0, not NaN) -> e4m3 byte, RNE, saturating to
    0x7E (448) above the largest finite value."""
    sigma = np.asarray(sigma, dtype=np.float32)
    if np.isnan(sigma).any() or (np.signbit(sigma) & (sigma != 0)).any():
        raise ValueError("e4m3_encode expects non-negative, non-NaN scales")
    return _nearest_even_index(sigma, E4M3_VALUES).astype(np.uint8)


def e4m3_encode_up(sigma) -> np.ndarray:
    """fp32 scale sigma (>= 0, not NaN) -> the smallest e4m3 value >= sigma
    (round toward +inf), saturating to 0x7E (448) when sigma exceeds it.

    This is the "truncation-free" scale of the transposition-invariant 2D
    paper (abstract: "truncation-free scaling"): with s >= block_amax / 6 the
    largest element maps to at most 6, so no element is clipped.  The page
    gives no formula; rounding the scale up is the plainest reading.
    """
    sigma = np.asarray(sigma, dtype=np.float32)
    if np.isnan(sigma).any() or (np.signbit(sigma) & (sigma != 0)).any():
        raise ValueError("e4m3_encode_up expects non-negative, non-NaN scales")
    idx = np.searchsorted(E4M3_VALUES.astype(np.float64), sigma.astype(np.float64), side="left")
    return np.minimum(idx, len(E4M3_VALUES) - 1).astype(np.uint8)


def e2m1_rtn_index(v) -> np.ndarray:
    """Magnitude v (>= 0, not NaN) -> e2m1 magnitude index by RNE on the
    grid, saturating at 6 (index 7).  NaN handling is the caller's."""
    return _nearest_even_index(v, E2M1_GRID)


def e2m1_sr_index(v, u16) -> np.ndarray:
    """Stochastic rounding of magnitude v (>= 0, not NaN) on the e2m1 grid.

    fp4-train, Method: for v between two grid points lo <= v < hi the higher
    point is taken with probability equal to the fractional distance
    f = (v - lo) / (hi - lo).  Reading (the card fixes neither the draw nor
    the comparison): the uniform draw is u = u16 * 2**-16 and the value
    rounds up iff u < f22, where f22 is f truncated to 22 fractional bits.
    On [1, 6) f22 == f; below 1 the truncation moves the decision only when
    u sits within 2**-22 below f, so P(up) stays within 2**-22 of f (the
    16-bit draw alone already limits it to 2**-16).  v >= 6 saturates to 6
    with no draw.  Every step is exact in float32: v - lo by Sterbenz (or
    lo = 0), hi - lo is a power of two, and the truncation is a floor of f
    scaled by 2**22.
    """
    v = np.asarray(v, dtype=np.float32)
    u16 = np.asarray(u16)
    sat = v >= F32(6.0)
    vv = np.where(sat, F32(0.0), v)
    lo = np.searchsorted(E2M1_GRID, vv, side="right") - 1  # grid[lo] <= v < grid[lo+1]
    lo = np.clip(lo, 0, 6)
    g_lo = E2M1_GRID[lo]
    g_hi = E2M1_GRID[lo + 1]
    f = (vv - g_lo) / (g_hi - g_lo)
    f22 = np.floor(f * F32(2.0 ** 22)) * F32(2.0 ** -22)
    u = u16.astype(np.float32) * F32(2.0 ** -16)
    up = u < f22
    idx = lo + up.astype(np.int64)
    return np.where(sat, 7, idx).astype(np.int64)


def bf16_bits_to_f32(b) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact: the bits become the top
    half of the float32 pattern)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> uint16 bf16 bits, round-to-nearest-even; NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=np.float32)
    u = np.ascontiguousarray(x).view(np.uint32).astype(np.uint64).reshape(x.shape)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), r).astype(np.uint16)
