"""Pins for the oracle's number formats (CPU only).

Each check ties the oracle to something other than itself: the grid printed
on the fp4-train card, torch's float8_e4m3fn / bfloat16 casts (library
routines), exact rational enumeration, and byte values the e4m3 format fixes.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as fm
from tests.exact_f32 import E2M1, E4M3, exact, nearest_even

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.txt")


def page_values():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            k, *v = line.split()
            out[k] = [float(t) for t in v]
    return out


def test_e2m1_grid_is_the_pages_grid():
    assert np.array_equal(oracle.E2M1_GRID, np.array(page_values()["e2m1_grid"], np.float32))


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(127, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(oracle.E4M3_VALUES, ref)
    assert oracle.E4M3_VALUES[-1] == page_values()["e4m3_max"][0]
    assert np.all(np.diff(oracle.E4M3_VALUES) > 0)


@pytest.mark.parametrize("value,byte", [(1.0, 0x38), (256.0, 0x78), (384.0, 0x7C), (448.0, 0x7E),
                                        (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (0.0, 0x00)])
def test_e4m3_known_bytes(value, byte):
    assert int(oracle.e4m3_encode(np.float32(value))) == byte


def test_e4m3_ties_and_saturation():
    # 2**-10 is halfway between 0 and 2**-9: ties to the even code 0x00.
    assert int(oracle.e4m3_encode(np.float32(2.0 ** -10))) == 0x00
    assert int(oracle.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))) == 0x01
    # 3*2**-10 is halfway between 0x01 and 0x02: even -> 0x02.
    assert int(oracle.e4m3_encode(np.float32(3 * 2.0 ** -10))) == 0x02
    # satfinite: 462 (rounds down), 464 (tie between 448 and the next step), 500, inf.
    for v in (462.0, 464.0, 500.0, 1e30, np.inf):
        assert int(oracle.e4m3_encode(np.float32(v))) == 0x7E


def _midpoints_and_neighbours(table):
    t = table.astype(np.float64)
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    return np.concatenate([mids, up, dn, table])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(123)
    logu = np.float32(2.0) ** rng.uniform(-12, np.log2(448.0), 400_000).astype(np.float32)
    vals = np.concatenate([_midpoints_and_neighbours(oracle.E4M3_VALUES), logu,
                           rng.uniform(0, 448, 100_000).astype(np.float32),
                           rng.uniform(0, 2 ** -6, 100_000).astype(np.float32)])
    vals = vals[(vals >= 0) & (vals <= 448)]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(vals), ref)


def test_e4m3_encode_brute_force_exact():
    rng = np.random.default_rng(5)
    vals = np.concatenate([_midpoints_and_neighbours(oracle.E4M3_VALUES)[::7],
                           rng.uniform(0, 500, 300).astype(np.float32)])
    got = oracle.e4m3_encode(vals)
    for v, g in zip(vals, got):
        assert nearest_even(exact(v), E4M3) == int(g)


def test_e2m1_rtn_brute_force_exact():
    rng = np.random.default_rng(7)
    vals = np.concatenate([_midpoints_and_neighbours(oracle.E2M1_GRID),
                           rng.uniform(0, 7, 2000).astype(np.float32),
                           np.array([6.0, 6.5, 1e30, np.inf, 0.0, 1e-45], np.float32)])
    got = oracle.e2m1_rtn_index(vals)
    for v, g in zip(vals, got):
        want = 7 if np.isinf(v) else nearest_even(exact(v), E2M1)
        assert want == int(g), v


def test_e2m1_rtn_threshold_form_dense():
    # Closed form of RNE with ties to the even index on this grid: the
    # threshold at 0.25, 1.25, 2.5, 5 belongs to the lower value, the one at
    # 0.75, 1.75, 3.5 to the upper.  Checked on every float32 in [0, 8) whose
    # low 8 mantissa bits are zero, and on 2**16 floats around each midpoint.
    bits = np.arange(0, 0x41000000, 256, dtype=np.uint32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-2 ** 15, 2 ** 15)[None, :]).reshape(-1)
    v = np.concatenate([bits, near.astype(np.uint32)]).view(np.float32)
    want = ((v > 0.25).astype(int) + (v >= 0.75) + (v > 1.25) + (v >= 1.75) + (v > 2.5)
            + (v >= 3.5) + (v > 5.0))
    assert np.array_equal(oracle.e2m1_rtn_index(v), want)


def test_e2m1_sr_fraction_is_exact_and_brackets():
    rng = np.random.default_rng(11)
    v = rng.uniform(0, 6, 3000).astype(np.float32)
    for u16 in (0, 1, 32768, 65535):
        idx = oracle.e2m1_sr_index(v, np.full(v.shape, u16))
        for vi, ii in zip(v[:300], idx[:300]):
            x = exact(vi)
            lo = max(i for i, g in enumerate(E2M1) if g <= x)
            if E2M1[lo] == x:
                assert ii == lo  # on-grid values never move
                continue
            f = (x - E2M1[lo]) / (E2M1[lo + 1] - E2M1[lo])
            f22 = Fraction(math.floor(f * 2 ** 22), 2 ** 22)
            assert ii == (lo + 1 if Fraction(u16, 65536) < f22 else lo)
    sat = oracle.e2m1_sr_index(np.array([6.0, 7.0, np.inf], np.float32), np.zeros(3))
    assert list(sat) == [7, 7, 7]


def test_e2m1_sr_22_bit_fraction_boundaries():
    # Above 1 the fraction has exactly 22 bits, so the reading changes nothing
    # there; below 1 a draw just under the exact fraction but not under its
    # 22-bit truncation keeps the lower grid point.
    v = np.array([0x3F378F81], np.uint32).view(np.float32)  # 0.717..., odd last mantissa bit
    f = (exact(v[0]) - Fraction(1, 2)) / Fraction(1, 2)
    u = math.floor(f * 2 ** 16)
    assert Fraction(u, 2 ** 16) < f and Fraction(u, 2 ** 16) == Fraction(math.floor(f * 2 ** 22), 2 ** 22)
    assert oracle.e2m1_sr_index(v, np.array([u]))[0] == 1          # stays at 0.5
    assert oracle.e2m1_sr_index(v, np.array([u - 1]))[0] == 2      # rounds up to 1.0
    tiny = np.array([1e-10, 2.0 ** -24, 2.0 ** -23, 3 * 2.0 ** -25], np.float32)
    assert list(oracle.e2m1_sr_index(tiny, np.zeros(4))) == [0, 0, 1, 0]
    # on [1, 6) every fraction is representable in 22 bits: same as the exact rule
    rng = np.random.default_rng(2)
    w = rng.uniform(1, 6, 5000).astype(np.float32)
    uu = rng.integers(0, 65536, 5000)
    for vi, ui, ii in zip(w[:500], uu[:500], oracle.e2m1_sr_index(w, uu)[:500]):
        x = exact(vi)
        lo = max(i for i, g in enumerate(E2M1) if g <= x)
        f = (x - E2M1[lo]) / (E2M1[lo + 1] - E2M1[lo])
        assert f * 2 ** 22 == math.floor(f * 2 ** 22)
        assert ii == (lo + 1 if Fraction(int(ui), 65536) < f else lo)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    raw = rng.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = x[~np.isnan(x)]
    ties = (rng.integers(0, 2 ** 16, 10000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[~np.isnan(ties)],
                        np.array([3.4e38, -3.4e38, 1e-45, -0.0, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f32(ref).view(np.uint32), back.view(np.uint32))
    assert int(oracle.f32_to_bf16_bits(np.float32(np.nan))) == 0x7FC0
