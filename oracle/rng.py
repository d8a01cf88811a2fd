"""Counter-based random bits for stochastic rounding (oracle; test
infrastructure only).

fp4-train, Method: stochastic rounding draws from "a counter-based (seed,
step, global-index)" generator.  The pages fix nothing more, so the function
is this library's own choice, built from one published hash:

    H = the 32-bit "pcg" hash of Jarzynski & Olano, "Hash Functions for GPU
        Rendering", JCGT 9(3), 2020 - one step of the 32-bit PCG linear
        congruential generator (multiplier 747796405, increment 2891336453)
        followed by the PCG RXS-M-XS output permutation (multiplier
        277803737).

    key  = H(seed XOR H(step XOR 0x9E3779B9))
    For element i = m*K + k of a row-major [M, K] tensor (the global index),
    the pair index p = i >> 1 draws one word w = H(p XOR key); element i takes
    the 16-bit field u16 = (w >> (16 * (i & 1))) & 0xFFFF.

One hash therefore serves the two elements that share a packed byte.  H is a
bijection of the 32-bit integers, so within one (seed, step) no two pairs get
the same word.  Parity of these bits against the pages is unpinned (the
pages leave them open); tests/test_oracle_rng.py pins the structure and the
statistics.
"""
from __future__ import annotations

import numpy as np

_U32 = np.uint32
GOLDEN = 0x9E3779B9


def pcg_hash(v) -> np.ndarray:
    """Jarzynski & Olano's pcg hash, uint32 -> uint32 (wrapping arithmetic)."""
    v = np.asarray(v, dtype=np.uint32)
    with np.errstate(over="ignore"):
        state = v * _U32(747796405) + _U32(2891336453)
        word = ((state >> ((state >> _U32(28)) + _U32(4))) ^ state) * _U32(277803737)
    return (word >> _U32(22)) ^ word


def rng_key(seed: int, step: int) -> np.uint32:
    inner = pcg_hash(np.array([(step ^ GOLDEN) & 0xFFFFFFFF], dtype=np.uint32))[0]
    return pcg_hash(np.array([(seed & 0xFFFFFFFF) ^ int(inner)], dtype=np.uint32))[0]


def sr_u16(index, seed: int, step: int) -> np.ndarray:
    """16-bit uniform field for each global element index (int64 array)."""
    index = np.asarray(index, dtype=np.int64)
    if index.size and int(index.max()) >> 1 > 0xFFFFFFFF:
        raise ValueError("pair index exceeds 32 bits")
    key = rng_key(seed, step)
    p = (index >> 1).astype(np.uint32)
    w = pcg_hash(p ^ key)
    shift = ((index & 1) * 16).astype(np.uint32)
    return ((w >> shift) & _U32(0xFFFF)).astype(np.uint32)
