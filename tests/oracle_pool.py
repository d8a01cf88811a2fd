"""Run the CPU oracle over row chunks of a full-size tensor in a process
pool, so that GPU outputs can be compared with it on every row.

Workers are spawned (fresh interpreters that import numpy and the oracle
only, never the GPU runtime), at most 16 or the cores this process may use.
Rows are independent on every 1x16 path given the global amax, and 16-row
strips on the 16x16 paths; stochastic rounding takes each chunk's row offset,
so the chunks together are exactly the oracle on the whole tensor.
"""
from __future__ import annotations

import atexit
import multiprocessing as mp
import os

import numpy as np

_pool = None


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool():
    global _pool
    if _pool is None:
        _pool = mp.get_context("spawn").Pool(workers())
        atexit.register(_pool.terminate)
    return _pool


def row_chunks(M, multiple=1, per_worker=3):
    """Row ranges covering [0, M), each a multiple of `multiple` rows."""
    n = max(1, workers() * per_worker)
    step = max(multiple, (M // n + multiple - 1) // multiple * multiple)
    return [(r, min(r + step, M)) for r in range(0, M, step)]


def starmap(fn, args):
    return pool().starmap(fn, args)


def concat(results, axis=0):
    """Concatenate a list of result tuples field by field."""
    return tuple(np.concatenate(f, axis=axis[i] if isinstance(axis, tuple) else axis)
                 for i, f in enumerate(zip(*results)))
