"""The stochastic-rounding kernels form the draw words of N consecutive pairs
(N = 4 in the 2D pass, 2 in the 1x16 pass) from one shared LCG multiply:
for a first pair index p0 that is a multiple of N,

    ((p0 + j) ^ key) * A + C  ==  (p0 ^ (key & ~(N-1))) * A + (((key & (N-1)) ^ j) * A + C)   (mod 2^32)

for j = 0 .. N-1, where A and C are the multiplier and increment of the pcg
hash's LCG step (Jarzynski and Olano, "Hash Functions for GPU Rendering").
The output permutation is then applied to equal states, so the words equal
pcg_hash((p0 + j) ^ key).  This CPU test checks the identity over every
low-bit pattern of the key and pair indices spread over the 32-bit range,
including the wrap at 2^32."""
import numpy as np
import pytest

from oracle.rng import pcg_hash

A = np.uint32(747796405)
C = np.uint32(2891336453)


def _states_direct(p0, key, n):
    return [((p0 + np.uint32(j)) ^ key) * A + C for j in range(n)]


def _states_grouped(p0, key, n):
    lo = np.uint32(n - 1)
    base = (p0 ^ (key & ~lo)) * A
    return [base + (((key & lo) ^ np.uint32(j)) * A + C) for j in range(n)]


@pytest.mark.parametrize("n", [2, 4])
def test_grouped_lcg_step_equals_direct(n):
    rng = np.random.default_rng(11)
    p0 = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    p0 &= ~np.uint32(n - 1)
    p0[:4] = np.array([0, 2**32 - n, 2**31 - n, n], dtype=np.uint32)  # ends and the wrap
    with np.errstate(over="ignore"):
        for key_hi in rng.integers(0, 2**32, size=8, dtype=np.uint64).astype(np.uint32):
            for low in range(n):
                key = (key_hi & ~np.uint32(n - 1)) | np.uint32(low)
                keys = np.full_like(p0, key)
                d = _states_direct(p0, keys, n)
                g = _states_grouped(p0, keys, n)
                for j in range(n):
                    assert np.array_equal(d[j], g[j]), (n, int(key), j)


def test_grouped_words_match_the_hash():
    """The index form behind the identity, (p0 + j) ^ key ==
    (p0 ^ (key & ~3)) + ((key & 3) ^ j) for p0 a multiple of four, and the
    full hash of the grouped state against pcg_hash of the direct index."""
    rng = np.random.default_rng(12)
    p0 = (rng.integers(0, 2**32, size=4096, dtype=np.uint64).astype(np.uint32)) & ~np.uint32(3)
    with np.errstate(over="ignore"):
        for key in (np.uint32(0), np.uint32(1), np.uint32(2), np.uint32(3), np.uint32(0xDEADBEEF)):
            for j in range(4):
                want = pcg_hash((p0 + np.uint32(j)) ^ key)
                st = _states_grouped(p0, np.full_like(p0, key), 4)[j]
                v = (p0 ^ (key & ~np.uint32(3))) + ((key & np.uint32(3)) ^ np.uint32(j))
                assert np.array_equal(v, (p0 + np.uint32(j)) ^ key)
                assert np.array_equal(v * A + C, st)
                assert np.array_equal(pcg_hash(v), want)
