"""GPU vs CPU-oracle parity at the five workloads' full sizes, through the C
ABI, in the launch configuration the benchmark times.

The oracle cannot run every full-size case whole in seconds, so each test
runs the GPU over the whole tensor and compares sampled rows (or 16-row
strips for 16x16 tiles) bit for bit.  This is exact because, given the
global amax (compared in full), rows are independent on every 1x16 path and
16-row strips are independent on the 16x16 paths; the oracle is told each
sample's row offset so stochastic rounding draws the same random numbers.

Workloads (inputs from workloads.py):
* 256x256 fp32 N(0,1): quantize / dequantize / qdq, RTN and SR (whole tensor).
* 4096x4096 stored weight with error feedback: three full-size steps with
  sampled rows, and the 500-step trajectory of a 32-row slice.
* 8192x7168 bf16 row-scaled four-over-six, MAE and MSE, bound 256.
* 7168x18432 bf16 16x16 with SR and a per-tensor amax (two-pass), plus the
  truncation-free scale, four-over-six on 16x16 tiles and the fused
  row + column 1x16 quantization on the same tensor.
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
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@functools.lru_cache(maxsize=None)
def _input(name):
    return getattr(workloads, name)()


def _sample_rows(M, n=48, seed=0):
    r = np.random.default_rng(seed).choice(M, n, replace=False)
    return np.unique(np.concatenate([np.arange(16), r, [M - 1]]))


def _sample_strips(M, seed=0):
    ns = M // 16
    s = np.random.default_rng(seed).choice(ns, 3, replace=False)
    return np.unique(np.concatenate([[0, ns - 1], s]))


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


def _ef_x(W_bits_or_f32, g):
    """x_t = W_t - 1e-4 * g_t in fp32, two separate roundings (caller side)."""
    return W_bits_or_f32 - np.float32(workloads.EF_LR) * g


@pytest.mark.parametrize("sr", [False, True], ids=["rtn_ef", "sr_ef"])
def test_ef_weight_full_size_steps(sr):
    M, K = workloads.EF_SHAPE
    W0 = _input("ef_weight0")
    rows = _sample_rows(M)
    Wd = to_dev(W0).float()
    r = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    Ws = oracle.bf16_bits_to_f32(W0[rows])
    rs = np.zeros((len(rows), K), np.float32)
    for t in range(3):
        g = workloads.ef_grad(t)
        gd = torch.from_numpy(g).cuda()
        xd = Wd - gd * np.float32(workloads.EF_LR)
        out = nv.qdq(xd, stochastic=sr, residual=r, seed=0, step=t)
        xs = _ef_x(Ws, g[rows])
        wo = np.empty((len(rows), K), np.uint16)
        for i, m in enumerate(rows):  # row offsets differ; rows are independent
            rr = rs[i:i + 1]
            wo[i] = oracle.qdq(xs[i:i + 1], stochastic=sr, residual=rr, seed=0, step=t, row_offset=int(m))[0]
        assert_bitwise(to_np(out)[rows], wo, f"W step {t}")
        assert_bitwise(to_np(r)[rows], rs, f"residual step {t}")
        Wd = out.float()
        Ws = oracle.bf16_bits_to_f32(wo)


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


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_act_rows_four_over_six_full_size(err):
    x = _input("act_rows_input")
    M, K = x.shape
    xd = to_dev(x)
    p, s, A = nv.quantize_4over6(xd, None, err_mode=err, e4m3_scale_bound=256, row_scaled=True)
    assert_bitwise(to_np(A), oracle.amax(x, mode="row"), "row amax (all rows)")
    rows = _sample_rows(M, 64, seed=1)
    wp, ws = oracle.quantize_4over6(x[rows], to_np(A)[rows], err_mode=err, bound=256.0)
    assert_bitwise(to_np(s)[rows], ws, "scales")
    assert_bitwise(to_np(p)[rows], wp, "codes")
    # the same rows with the amax vector given instead of computed
    p2, s2, _ = nv.quantize_4over6(xd, A, err_mode=err, e4m3_scale_bound=256, row_scaled=True)
    assert_bitwise(to_np(p2)[rows], wp, "codes (amax given)")
    assert_bitwise(to_np(s2)[rows], ws, "scales (amax given)")


def test_act_rows_four_over_six_every_row():
    """The metric workload (8192x7168 bf16, row amax computed in the pass,
    MAE, bound 256) against the oracle on every row, not a sample."""
    x = _input("act_rows_input")
    p, s, A = nv.quantize_4over6(to_dev(x), None, err_mode="mae", e4m3_scale_bound=256, row_scaled=True)
    wA = oracle.amax(x, mode="row")
    assert_bitwise(to_np(A), wA, "row amax")
    wp, ws = oracle.quantize_4over6(x, wA, err_mode="mae", bound=256.0)
    assert_bitwise(to_np(s), ws, "scales (every row)")
    assert_bitwise(to_np(p), wp, "codes (every row)")


def _weight_2d():
    x = _input("weight_2d_input")
    xd = to_dev(x)
    A = nv.amax(xd, mode="tensor")
    assert_bitwise(to_np(A), np.array([oracle.amax(x)], np.float32), "per-tensor amax")
    return x, xd, A


@pytest.mark.parametrize("tf", [False, True], ids=["nearest", "truncfree"])
def test_weight_2d_sr_full_size(tf):
    x, xd, A = _weight_2d()
    M, K = x.shape
    pr, pc, ts = nv.quantize_2d(xd, A, stochastic=True, seed=0, step=0, truncation_free=tf)
    pr, pc, ts = to_np(pr), to_np(pc), to_np(ts)
    Af = np.float32(to_np(A)[0])
    for st in _sample_strips(M):
        r0 = int(st) * 16
        wr, wc, wt = oracle.quantize_2d(x[r0:r0 + 16], stochastic=True, seed=0, step=0, global_amax=Af,
                                        row_offset=r0, truncation_free=tf)
        assert_bitwise(ts[st:st + 1], wt, f"tile scales strip {st}")
        assert_bitwise(pr[r0:r0 + 16], wr, f"rowwise strip {st}")
        assert_bitwise(pc[:, r0 // 2:r0 // 2 + 8], wc, f"columnwise strip {st}")


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_weight_2d_four_over_six_tiles_full_size(err):
    x, xd, A = _weight_2d()
    M, K = x.shape
    pr, pc, ts = nv.quantize_4over6_2d(xd, A, err_mode=err, e4m3_scale_bound=256)
    pr, pc, ts = to_np(pr), to_np(pc), to_np(ts)
    Af = np.float32(to_np(A)[0])
    for st in _sample_strips(M, seed=1):
        r0 = int(st) * 16
        wr, wc, wt = oracle.quantize_4over6_2d(x[r0:r0 + 16], Af, err_mode=err, bound=256.0)
        assert_bitwise(ts[st:st + 1], wt, f"tile scales strip {st}")
        assert_bitwise(pr[r0:r0 + 16], wr, f"rowwise strip {st}")
        assert_bitwise(pc[:, r0 // 2:r0 // 2 + 8], wc, f"columnwise strip {st}")


@pytest.mark.parametrize("fos", [False, True], ids=["standard", "four_over_six"])
def test_weight_2d_rowcol_full_size(fos):
    x, xd, A = _weight_2d()
    M, K = x.shape
    got = [to_np(t) for t in nv.quantize_rowcol(xd, A, four_over_six=fos)]
    Af = np.float32(to_np(A)[0])
    bound = 256.0 if fos else 448.0
    for st in _sample_strips(M, seed=2):
        r0 = int(st) * 16
        wpr, wsr, wpc, wsc = oracle.quantize_rowcol(x[r0:r0 + 16], Af, four_over_six=fos, bound=bound)
        assert_bitwise(got[0][r0:r0 + 16], wpr, f"row codes strip {st}")
        assert_bitwise(got[1][r0:r0 + 16], wsr, f"row scales strip {st}")
        assert_bitwise(got[2][:, r0 // 2:r0 // 2 + 8], wpc, f"col codes strip {st}")
        assert_bitwise(got[3][:, st:st + 1], wsc, f"col scales strip {st}")


@pytest.mark.parametrize("r0_kind", ["zeros", "normal"])
def test_heavy_qdq_sr_ef_full_size(r0_kind):
    x = _input("heavy_input")
    M, K = x.shape
    r0 = np.zeros((M, K), np.float32) if r0_kind == "zeros" else _input("heavy_residual")
    rows = _sample_rows(M, 64, seed=3)
    rs = r0[rows].copy()
    r = torch.from_numpy(r0).cuda()
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    L.check(L.lib().nvfp4_qdq(to_dev(x).data_ptr(), L.BF16, M, K, r.data_ptr(), None, L.SR,
                              workloads.HEAVY_SEED, workloads.HEAVY_STEP, out.data_ptr(), L.BF16,
                              None, None, torch.cuda.current_stream().cuda_stream), "qdq")
    wo = np.empty((len(rows), K), np.uint16)
    for i, m in enumerate(rows):
        wo[i] = oracle.qdq(x[m:m + 1], stochastic=True, residual=rs[i:i + 1], seed=workloads.HEAVY_SEED,
                           step=workloads.HEAVY_STEP, row_offset=int(m))[0]
    assert_bitwise(to_np(out)[rows], wo, "qdq out")
    assert_bitwise(to_np(r)[rows], rs, "residual")
