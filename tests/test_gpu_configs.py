"""GPU vs CPU-oracle parity at the five workloads' full sizes, through the C
ABI, in the launch configuration the benchmark times, on every row, strip
and output byte (the four-over-six pull request compares whole outputs:
Bitwise validation).

The oracle runs over row chunks in a process pool (tests/oracle_pool.py).
This is exact: given the global amax (compared in full), rows are
independent on every 1x16 path and 16-row strips on the 16x16 paths, and
stochastic rounding is told each chunk's row offset so it draws the same
numbers.

Workloads (inputs from workloads.py):
* 256x256 fp32 N(0,1): quantize / dequantize / qdq, RTN and SR.
* 4096x4096 stored weight with error feedback (RTN and SR): the whole tensor
  at steps 0, 1 and 499 of the 500-step trajectory, and every 50th step of
  a 32-row slice's own 500-step oracle trajectory.
* 8192x7168 bf16 row-scaled four-over-six, MAE and MSE, bound 256, with the
  row amax computed in the pass and given; the row-scaled dequantize.
* 7168x18432 bf16 16x16 with SR and a per-tensor amax (two-pass), plus the
  truncation-free scale, four-over-six on 16x16 tiles (MAE, MSE) and the
  fused row + column 1x16 quantization (standard, four-over-six).
* 16384x8192 bf16 heavy-tailed qdq with SR + EF, seed 7, step 123, residual
  zero and 0.01 * N(0,1).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
import fp4_block_quantization_nvfp4_amd as nv
from fp4_block_quantization_nvfp4_amd import _lib as L
from tests import oracle_pool as P
from tests import pool_tasks as T
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@functools.lru_cache(maxsize=None)
def _input(name):
    return getattr(workloads, name)()


def test_small_256x256():
    x = workloads.small_input()
    xd = to_dev(x)
    for sr in (False, True):
        wp, ws = oracle.quantize(x, stochastic=sr, seed=0, step=0)
        p, s = nv.quantize(xd, stochastic=sr, seed=0, step=0)
        assert_bitwise(to_np(p), wp, f"codes sr={sr}")
        assert_bitwise(to_np(s), ws, f"scales sr={sr}")
        want = oracle.dequantize(wp, ws, 256, 256)
        assert_bitwise(to_np(nv.dequantize(p, s, 256, 256)), want, f"dequant sr={sr}")
        wo = oracle.qdq(x, stochastic=sr)[0]
        assert_bitwise(to_np(nv.qdq(xd, stochastic=sr)), wo, f"qdq sr={sr}")


def _ef_x(W_f32, g):
    """x_t = W_t - 1e-4 * g_t in fp32, two separate roundings (caller side)."""
    return W_f32 - np.float32(workloads.EF_LR) * g


def _oracle_qdq_full(x, r, sr, seed, step):
    """The oracle's qdq + EF step on the whole tensor: (bf16 out, new r)."""
    M = x.shape[0]
    res = P.starmap(T.qdq, [(x[a:b], r[a:b], sr, seed, step, a) for a, b in P.row_chunks(M)])
    return np.concatenate([t[0] for t in res]), np.concatenate([t[3] for t in res])


def test_ef_weight_full_tensor_steps():
    """Whole-tensor parity, RTN + EF and SR + EF side by side on the same
    gradients, at steps 0, 1 (from the oracle's own trajectory) and 499 (the
    oracle's step applied to the GPU's state after 499 steps; the 500-step
    trajectory itself is compared on a slice below)."""
    M, K = workloads.EF_SHAPE
    W0 = _input("ef_weight0")
    modes = (False, True)
    Wd = {sr: to_dev(W0).float() for sr in modes}
    r = {sr: torch.zeros((M, K), dtype=torch.float32, device="cuda") for sr in modes}
    Ws = {sr: oracle.bf16_bits_to_f32(W0) for sr in modes}
    rs = {sr: np.zeros((M, K), np.float32) for sr in modes}
    last = workloads.EF_STEPS - 1
    pending = []  # gradients of the next steps, drawn by the pool in windows of 32 steps
    for t in range(workloads.EF_STEPS):
        if t < 2:
            g = workloads.ef_grad(t)
        else:
            if not pending:
                pending = P.starmap(T.ef_grad, [(u,) for u in range(t, min(t + 32, workloads.EF_STEPS))])
            g = pending.pop(0)
        gd = torch.from_numpy(g).cuda()
        for sr in modes:
            xd = Wd[sr] - gd * np.float32(workloads.EF_LR)
            if t == last:
                xs, rs[sr] = to_np(xd), to_np(r[sr]).copy()
            elif t < 2:
                xs = _ef_x(Ws[sr], g)
            out = nv.qdq(xd, stochastic=sr, residual=r[sr], seed=0, step=t)
            if t < 2 or t == last:
                wo, rs[sr] = _oracle_qdq_full(xs, rs[sr], sr, 0, t)
                what = f"{'SR' if sr else 'RTN'} step {t} (whole tensor)"
                assert_bitwise(to_np(out), wo, f"W {what}")
                assert_bitwise(to_np(r[sr]), rs[sr], f"residual {what}")
                Ws[sr] = oracle.bf16_bits_to_f32(wo)
            Wd[sr] = out.float()


@pytest.mark.parametrize("sr", [False, True], ids=["rtn_ef", "sr_ef"])
def test_ef_weight_500_steps_row_slice(sr):
    rows, K = 32, workloads.EF_SHAPE[1]
    W0 = _input("ef_weight0")[:rows]
    Wd = to_dev(W0).float()
    r = torch.zeros((rows, K), dtype=torch.float32, device="cuda")
    Ws = oracle.bf16_bits_to_f32(W0)
    rs = np.zeros((rows, K), np.float32)
    for t in range(workloads.EF_STEPS):
        g = workloads.ef_grad(t, rows=rows)
        xd = Wd - torch.from_numpy(g).cuda() * np.float32(workloads.EF_LR)
        out = nv.qdq(xd, stochastic=sr, residual=r, seed=0, step=t)
        wo = oracle.qdq(_ef_x(Ws, g), stochastic=sr, residual=rs, seed=0, step=t)[0]
        if t % 50 == 0 or t == workloads.EF_STEPS - 1:
            assert_bitwise(to_np(out), wo, f"W step {t}")
            assert_bitwise(to_np(r), rs, f"residual step {t}")
        Wd = out.float()
        Ws = oracle.bf16_bits_to_f32(wo)
    assert_bitwise(to_np(out), wo, "final W")


def _oracle_4over6_rows(x, A, err):
    res = P.starmap(T.four_over_six, [(x[a:b], A[a:b], err, 256.0) for a, b in P.row_chunks(x.shape[0])])
    return P.concat(res)


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_act_rows_four_over_six_every_row(err):
    """The metric workload (8192x7168 bf16, bound 256, row amax computed in
    the pass, and given) against the oracle on every row."""
    x = _input("act_rows_input")
    xd = to_dev(x)
    p, s, A = nv.quantize_4over6(xd, None, err_mode=err, e4m3_scale_bound=256, row_scaled=True)
    wA = oracle.amax(x, mode="row")
    assert_bitwise(to_np(A), wA, "row amax (every row)")
    wp, ws = _oracle_4over6_rows(x, wA, err)
    assert_bitwise(to_np(s), ws, "scales (every row)")
    assert_bitwise(to_np(p), wp, "codes (every row)")
    p2, s2, _ = nv.quantize_4over6(xd, A, err_mode=err, e4m3_scale_bound=256, row_scaled=True)
    assert_bitwise(to_np(s2), ws, "scales (amax given, every row)")
    assert_bitwise(to_np(p2), wp, "codes (amax given, every row)")
    if err == "mae":
        # the row-scaled dequantize of these outputs, every element
        M, K = x.shape
        got = nv.dequantize(p, s, M, K, global_amax=A, row_scaled=True, bound=256.0)
        res = P.starmap(T.dequantize, [(wp[a:b], ws[a:b], b - a, K, wA[a:b], 256.0, "row")
                                       for a, b in P.row_chunks(M)])
        assert_bitwise(to_np(got), P.concat(res)[0], "row-scaled dequantize (every element)")


def _weight_2d():
    x = _input("weight_2d_input")
    xd = to_dev(x)
    A = nv.amax(xd, mode="tensor")
    assert_bitwise(to_np(A), np.array([oracle.amax(x)], np.float32), "per-tensor amax")
    return x, xd, A, np.float32(to_np(A)[0])


@pytest.mark.parametrize("tf", [False, True], ids=["nearest", "truncfree"])
def test_weight_2d_sr_every_strip(tf):
    x, xd, A, Af = _weight_2d()
    M, K = x.shape
    pr, pc, ts = nv.quantize_2d(xd, A, stochastic=True, seed=0, step=0, truncation_free=tf)
    res = P.starmap(T.quantize_2d, [(x[a:b], Af, True, 0, 0, a, tf) for a, b in P.row_chunks(M, 16)])
    wr, wc, wt = P.concat(res, axis=(0, 1, 0))
    assert_bitwise(to_np(ts), wt, "tile scales (every tile)")
    assert_bitwise(to_np(pr), wr, "rowwise codes (every strip)")
    assert_bitwise(to_np(pc), wc, "columnwise codes (every strip)")


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_weight_2d_four_over_six_tiles_every_strip(err):
    x, xd, A, Af = _weight_2d()
    M, K = x.shape
    pr, pc, ts = nv.quantize_4over6_2d(xd, A, err_mode=err, e4m3_scale_bound=256)
    res = P.starmap(T.four_over_six_2d, [(x[a:b], Af, err, 256.0) for a, b in P.row_chunks(M, 16)])
    wr, wc, wt = P.concat(res, axis=(0, 1, 0))
    assert_bitwise(to_np(ts), wt, "tile scales (every tile)")
    assert_bitwise(to_np(pr), wr, "rowwise codes (every strip)")
    assert_bitwise(to_np(pc), wc, "columnwise codes (every strip)")


@pytest.mark.parametrize("fos,err", [(False, "mae"), (True, "mae"), (True, "mse")],
                         ids=["standard", "four_over_six", "four_over_six_mse"])
def test_weight_2d_rowcol_every_block(fos, err):
    x, xd, A, Af = _weight_2d()
    M, K = x.shape
    got = [to_np(t) for t in nv.quantize_rowcol(xd, A, four_over_six=fos, err_mode=err)]
    bound = 256.0 if fos else 448.0
    res = P.starmap(T.rowcol, [(x[a:b], Af, fos, err, bound) for a, b in P.row_chunks(M, 16)])
    want = P.concat(res, axis=(0, 0, 1, 1))
    for g, w, what in zip(got, want, ("row codes", "row scales", "col codes", "col scales")):
        assert_bitwise(g, w, f"{what} (every block)")


@pytest.mark.parametrize("r0_kind", ["zeros", "normal"])
def test_heavy_qdq_sr_ef_every_row(r0_kind):
    x = _input("heavy_input")
    M, K = x.shape
    r0 = np.zeros((M, K), np.float32) if r0_kind == "zeros" else _input("heavy_residual")
    r = torch.from_numpy(r0).cuda()
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    L.check(L.lib().nvfp4_qdq(to_dev(x).data_ptr(), L.BF16, M, K, r.data_ptr(), None, L.SR,
                              workloads.HEAVY_SEED, workloads.HEAVY_STEP, out.data_ptr(), L.BF16,
                              None, None, torch.cuda.current_stream().cuda_stream), "qdq")
    res = P.starmap(T.qdq, [(x[a:b], r0[a:b], True, workloads.HEAVY_SEED, workloads.HEAVY_STEP, a)
                            for a, b in P.row_chunks(M)])
    assert_bitwise(to_np(out), np.concatenate([t[0] for t in res]), "qdq out (every row)")
    assert_bitwise(to_np(r), np.concatenate([t[3] for t in res]), "residual (every row)")
