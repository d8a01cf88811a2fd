"""Structure and statistics of the stochastic-rounding generator (CPU only).

The pages fix only that the generator is counter-based over (seed, step,
global index) (fp4-train, Method).  The exact bits are this library's choice,
so they are parity unpinned against the pages; these tests pin what a
plausible mistake would break: the hash is a bijection, the draws are
deterministic in (seed, step, index), the two elements of a pair read the two
halves of one word, and the 16-bit fields are uniform and uncorrelated.
"""
import numpy as np

import oracle


def test_pcg_hash_is_a_bijection_on_a_large_slice():
    v = np.arange(0, 1 << 22, dtype=np.uint32)
    for base in (0, 0x7FC00000, 0xFFC00000):
        h = oracle.pcg_hash(v + np.uint32(base))
        assert np.unique(h).size == v.size


def test_pcg_hash_wraps_like_unbounded_integers_mod_2_32():
    # numpy's uint32 arithmetic (and its shift-by-array promotion) must agree
    # with the same definition evaluated on Python's unbounded integers
    # reduced mod 2**32: one PCG32 LCG step, then the RXS-M-XS permutation.
    a, c = 747796405, 2891336453
    for v in (0, 1, 2, 12345, 0xFFFFFFFF, 0xDEADBEEF):
        s = (v * a + c) & 0xFFFFFFFF
        word = (((s >> ((s >> 28) + 4)) ^ s) * 277803737) & 0xFFFFFFFF
        assert int(oracle.pcg_hash(np.array([v], np.uint32))[0]) == (word >> 22) ^ word


def test_counter_based_determinism_and_pairing():
    idx = np.arange(0, 4096, dtype=np.int64) + 10 ** 9
    a = oracle.sr_u16(idx, seed=3, step=9)
    b = oracle.sr_u16(idx[::-1], seed=3, step=9)[::-1]
    assert np.array_equal(a, b)  # depends on the index only, not on order
    key = oracle.rng_key(3, 9)
    w = oracle.pcg_hash((idx[0::2] >> 1).astype(np.uint32) ^ key)
    assert np.array_equal(a[0::2], w & 0xFFFF)
    assert np.array_equal(a[1::2], w >> 16)
    assert not np.array_equal(a, oracle.sr_u16(idx, seed=4, step=9))
    assert not np.array_equal(a, oracle.sr_u16(idx, seed=3, step=10))


def _chi2_uniform(x, bins):
    counts = np.bincount(x, minlength=bins)
    exp = x.size / bins
    return float(((counts - exp) ** 2 / exp).sum())


def test_u16_fields_are_uniform():
    n = 1 << 22
    for seed, step in ((0, 0), (7, 123), (0, 499)):
        u = oracle.sr_u16(np.arange(n, dtype=np.int64), seed, step)
        # top 8 bits and low 8 bits: chi-square with 255 dof (mean 255, sd 22.6)
        for field in (u >> 8, u & 0xFF):
            c2 = _chi2_uniform(field.astype(np.int64), 256)
            assert 150 < c2 < 380, (seed, step, c2)
        # every bit near one half
        bits = ((u[:, None] >> np.arange(16)) & 1).mean(axis=0)
        assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / np.sqrt(n))


def test_u16_neighbours_and_steps_uncorrelated():
    n = 1 << 20
    i = np.arange(n, dtype=np.int64)
    u0 = oracle.sr_u16(i, 0, 0).astype(np.float64)
    u1 = oracle.sr_u16(i, 0, 1).astype(np.float64)
    for a, b in ((u0[:-1], u0[1:]), (u0[:-2], u0[2:]), (u0, u1)):
        r = np.corrcoef(a, b)[0, 1]
        assert abs(r) < 5 / np.sqrt(n)
