"""The four-over-six pull request's validation matrix, bit for bit against
the oracle (Validation (GB200, SM100) and CuTe DSL kernel - Bitwise
validation):

{mae, mse} x {bound 256, 448} x {1x16 per-tensor, 1x16 row-scaled, 16x16
per-tensor} x {bf16, fp32} x shapes, with rowwise and columnwise outputs
(the 1x16 per-tensor case also runs the fused row + column pass; 16x16 tiles
emit both), over

* the DSL kernel's shapes 128x256, 256x512, 64x1024, 128x320 with 16 seeds
  and 2048x7168 with 4 seeds (its oracle is ~60x the others' cost);
* the TE comparison's other shapes 128x128, 2048x1024, 304x304 with 4 seeds;

plus a 64-seed stress of the tightest case.  Inputs: N(0,1); odd seeds scale
each row by 2^u, u ~ U(-20, 20) (the wide dynamic range the pages list among
their special values).  The tightest case is the one whose blocks came
closest to a tie over the 16-seed matrix at 256x512 (a relative gap
|E4 - E6| / (E4 + E6) of 3e-8, about one ulp, with 29% exact ties): 1x16
per-tensor, MAE, bound 256, bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import fp4_block_quantization_nvfp4_amd as nv
from tests import oracle_pool as P
from tests import pool_tasks as T
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

SHAPES = [((128, 256), 16), ((256, 512), 16), ((64, 1024), 16), ((128, 320), 16), ((2048, 7168), 4),
          ((128, 128), 4), ((2048, 1024), 4), ((304, 304), 4)]
CASES = [("1x16", "tensor"), ("1x16", "row"), ("16x16", "tensor")]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _x(seed, M, K, dt):
    rng = np.random.default_rng([seed, M, K])
    x = rng.standard_normal((M, K), dtype=np.float32)
    if seed % 2:
        x *= np.exp2(rng.uniform(-20, 20, (M, 1))).astype(np.float32)
    return workloads.bf16_bits(x) if dt == "bf16" else x


def _oracle(fn, x, *args, multiple=1, axes=0):
    """The oracle on the whole tensor, in the pool when it is large."""
    M = x.shape[0]
    if x.size < (1 << 20):
        return fn(x, *args)
    res = P.starmap(fn, [(x[a:b],) + tuple(a_[a:b] if isinstance(a_, np.ndarray) and a_.ndim == 1 else a_
                                            for a_ in args) for a, b in P.row_chunks(M, multiple)])
    return P.concat(res, axis=axes)


def run_case(seed, M, K, err, bound, block, mode, dt):
    x = _x(seed, M, K, dt)
    xd = to_dev(x)
    what = f"seed={seed} {M}x{K} {err} {bound} {block} {mode} {dt}"
    if block == "1x16" and mode == "row":
        p, s, A = nv.quantize_4over6(xd, None, err_mode=err, e4m3_scale_bound=int(bound), row_scaled=True)
        wA = oracle.amax(x, mode="row")
        assert_bitwise(to_np(A), wA, f"row amax {what}")
        wp, ws = _oracle(T.four_over_six, x, wA, err, bound)
        assert_bitwise(to_np(s), ws, f"scales {what}")
        assert_bitwise(to_np(p), wp, f"codes {what}")
        return
    A = nv.amax(xd, mode="tensor")
    wA = oracle.amax(x)
    assert_bitwise(to_np(A), np.array([wA], np.float32), f"tensor amax {what}")
    if block == "1x16":
        p, s, _ = nv.quantize_4over6(xd, A, err_mode=err, e4m3_scale_bound=int(bound), row_scaled=False)
        got = [to_np(t) for t in nv.quantize_rowcol(xd, A, four_over_six=True, err_mode=err,
                                                     e4m3_scale_bound=int(bound))]
        want = _oracle(T.rowcol, x, wA, True, err, bound, multiple=16, axes=(0, 0, 1, 1))
        assert_bitwise(to_np(s), want[1], f"scales {what}")
        assert_bitwise(to_np(p), want[0], f"codes {what}")
        for g, w, nm in zip(got, want, ("row codes", "row scales", "col codes", "col scales")):
            assert_bitwise(g, w, f"rowcol {nm} {what}")
    else:
        r, c, ts = nv.quantize_4over6_2d(xd, A, err_mode=err, e4m3_scale_bound=int(bound))
        wr, wc, wt = _oracle(T.four_over_six_2d, x, wA, err, bound, multiple=16, axes=(0, 1, 0))
        assert_bitwise(to_np(ts), wt, f"tile scales {what}")
        assert_bitwise(to_np(r), wr, f"rowwise {what}")
        assert_bitwise(to_np(c), wc, f"columnwise {what}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("block,mode", CASES, ids=["1x16-tensor", "1x16-row", "16x16-tensor"])
@pytest.mark.parametrize("bound", [256.0, 448.0])
@pytest.mark.parametrize("err", ["mae", "mse"])
@pytest.mark.parametrize("shape,seeds", SHAPES, ids=[f"{m}x{k}" for (m, k), _ in SHAPES])
def test_validation_matrix(shape, seeds, err, bound, block, mode, dt):
    M, K = shape
    for seed in range(seeds):
        run_case(seed, M, K, err, bound, block, mode, dt)


def test_stress_tightest_case_64_seeds():
    for seed in range(64):
        run_case(1000 + seed, 256, 512, "mae", 256.0, "1x16", "tensor", "bf16")
