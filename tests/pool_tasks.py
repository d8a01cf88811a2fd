"""Oracle tasks executed by the spawned workers of tests/oracle_pool.py
(module-level functions, so they can be pickled by name).  Each returns the
oracle's outputs for one chunk of rows of a larger tensor."""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def four_over_six(x, A, err, bound, block="1x16"):
    return oracle.quantize_4over6(x, A, err_mode=err, bound=bound, block=block)


def four_over_six_2d(x, A, err, bound):
    return oracle.quantize_4over6_2d(x, A, err_mode=err, bound=bound)


def quantize_2d(x, A, stochastic, seed, step, row_offset, truncation_free):
    return oracle.quantize_2d(x, stochastic=stochastic, seed=seed, step=step, global_amax=A,
                              row_offset=row_offset, truncation_free=truncation_free)


def rowcol(x, A, fos, err, bound):
    return oracle.quantize_rowcol(x, A, four_over_six=fos, err_mode=err, bound=bound)


def qdq(x, r, stochastic, seed, step, row_offset, out="bf16"):
    r = None if r is None else np.array(r, np.float32, copy=True)
    o, p, s = oracle.qdq(x, stochastic=stochastic, residual=r, seed=seed, step=step, out=out,
                         row_offset=row_offset)
    return (o, p, s) if r is None else (o, p, s, r)


def dequantize(packed, scales, M, K, A, bound, scale_mode):
    return (oracle.dequantize(packed, scales, M, K, global_amax=A, scale_mode=scale_mode, bound=bound),)


def ef_grad(step):
    return workloads.ef_grad(step)
