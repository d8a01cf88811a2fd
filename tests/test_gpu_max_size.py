"""Every entry point at the largest accepted tensor, M * K = 2^33 elements
(fp4-train card, Requirements and limits: any M with K a multiple of 16; the
library's cap keeps the stochastic-rounding pair index within 32 bits).

Inputs are drawn on the device in row chunks from a seeded torch generator:
N(0,1) rows times a log-uniform per-row std 10^(4u - 2), as the row-scaled
activation workload.  Per-tensor tests plant one element 2^15 past element
2^32, so the two-pass amax must return exactly 2^15.  Each test compares
sampled 16-row strips with the oracle bit for bit: the first and last strips,
the strips on both sides of elements 2^31, 2^32 and 3 * 2^31 (where 32-bit
element or pair indices would wrap), and random strips.  Stochastic rounding
is checked at the global element indices of the strip (the oracle's
row_offset)."""
import numpy as np
import pytest
import torch

import oracle
import fp4_block_quantization_nvfp4_amd as nv
from tests.gpu_util import assert_bitwise, need_gpu, to_np

pytestmark = pytest.mark.gpu

N_ELEMS = 1 << 33
PLANT = 32768.0
SEED, STEP = 77, 5


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _need_free(gib):
    free, _ = torch.cuda.mem_get_info()
    if free < gib * (1 << 30):
        pytest.skip(f"needs {gib} GiB of free device memory, {free / (1 << 30):.0f} GiB free")


def _rows_input(M, K, seed, dtype=torch.bfloat16, chunk_elems=1 << 28):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.empty((M, K), dtype=dtype, device="cuda")
    step = max(1, chunk_elems // K)
    for r0 in range(0, M, step):
        r1 = min(M, r0 + step)
        z = torch.randn((r1 - r0, K), generator=g, device="cuda", dtype=torch.float32)
        std = torch.pow(10.0, torch.rand((r1 - r0, 1), generator=g, device="cuda") * 4.0 - 2.0)
        x[r0:r1] = (z * std).to(dtype)
        del z
    return x


def _plant(x):
    """One element of 2^15 past element 2^32 (larger than any drawn value)."""
    M, K = x.shape
    idx = (1 << 32) + 123 * K + 37
    x.view(-1)[idx] = PLANT
    return idx // K


def _strips(M, K, seed, n_random=4):
    rows = {0, M - 16}
    for e in (1 << 31, 1 << 32, 3 << 31):
        r = e // K
        for s in (r - 16, r):
            if 0 <= s <= M - 16:
                rows.add(s - s % 16)
    rng = np.random.default_rng(seed)
    rows |= {int(16 * s) for s in rng.integers(0, M // 16, n_random)}
    return sorted(rows)


def _host(t):
    return to_np(t)


def test_max_size_amax_quantize_dequantize_bf16():
    M, K = N_ELEMS // 8192, 8192
    _need_free(48)
    x = _rows_input(M, K, 1)
    prow = _plant(x)
    A = nv.amax(x)
    assert float(A.item()) == PLANT
    Arow = nv.amax(x, mode="row")
    packed, scale = nv.quantize(x, stochastic=True, seed=SEED, step=STEP, global_amax=A)
    xh = nv.dequantize(packed, scale, M, K, global_amax=A, bound=448.0)
    torch.cuda.synchronize()
    Ah = np.float32(PLANT)
    for r in sorted(set(_strips(M, K, 2)) | {prow - prow % 16}):
        xs = _host(x[r:r + 16])
        assert_bitwise(_host(Arow[r:r + 16]), oracle.amax(xs, mode="row"), f"row amax @ {r}")
        wp, ws = oracle.quantize(xs, stochastic=True, seed=SEED, step=STEP, global_amax=Ah, row_offset=r)
        assert_bitwise(_host(scale[r:r + 16]), ws, f"scales @ {r}")
        assert_bitwise(_host(packed[r:r + 16]), wp, f"codes @ {r}")
        wd = oracle.dequantize(wp, ws, 16, K, global_amax=Ah, scale_mode="tensor", bound=448.0)
        assert_bitwise(_host(xh[r:r + 16]), wd, f"dequantized @ {r}")


def test_max_size_qdq_error_feedback_bf16():
    M, K = N_ELEMS // 8192, 8192
    _need_free(80)
    x = _rows_input(M, K, 3)
    prow = _plant(x)
    g = torch.Generator(device="cuda").manual_seed(4)
    res = torch.empty((M, K), dtype=torch.float32, device="cuda")
    step = (1 << 28) // K
    for r0 in range(0, M, step):
        res[r0:r0 + step] = 0.01 * torch.randn((min(M, r0 + step) - r0, K), generator=g, device="cuda")
    # the amax of x + r (the planted element dominates): the residual-reading
    # amax pass at full size
    idx = (1 << 32) + 123 * K + 37
    A = nv.amax(x, residual=res)
    Ah = np.float32(PLANT) + np.float32(res.view(-1)[idx].item())
    assert_bitwise(_host(A), np.array([Ah], dtype=np.float32), "amax of x + r")
    strips = sorted(set(_strips(M, K, 5)) | {prow - prow % 16})
    r_before = {r: _host(res[r:r + 16]) for r in strips}
    out, packed, scale = nv.qdq(x, stochastic=True, residual=res, seed=SEED, step=STEP,
                                global_amax=A, return_codes=True)
    torch.cuda.synchronize()
    for r in strips:
        xs = _host(x[r:r + 16])
        rr = r_before[r].copy()
        wo, wp, ws = oracle.qdq(xs, stochastic=True, residual=rr, seed=SEED, step=STEP,
                                global_amax=Ah, row_offset=r)
        assert_bitwise(_host(out[r:r + 16]), wo, f"qdq out @ {r}")
        assert_bitwise(_host(packed[r:r + 16]), wp, f"codes @ {r}")
        assert_bitwise(_host(scale[r:r + 16]), ws, f"scales @ {r}")
        assert_bitwise(_host(res[r:r + 16]), rr, f"residual @ {r}")


def test_max_size_four_over_six_row_scaled_bf16():
    """The row kernel (row amax in the pass), then the row-scaled dequantize."""
    M, K = N_ELEMS // 8192, 8192
    _need_free(48)
    x = _rows_input(M, K, 6)
    p, s, Ar = nv.quantize_4over6(x, err_mode="mae", e4m3_scale_bound=256, row_scaled=True)
    xh = nv.dequantize(p, s, M, K, global_amax=Ar, row_scaled=True, bound=256.0)
    torch.cuda.synchronize()
    for r in _strips(M, K, 7):
        xs = _host(x[r:r + 16])
        wA = oracle.amax(xs, mode="row")
        assert_bitwise(_host(Ar[r:r + 16]), wA, f"row amax @ {r}")
        wp, ws = oracle.quantize_4over6(xs, wA, err_mode="mae", bound=256.0)
        assert_bitwise(_host(s[r:r + 16]), ws, f"scales @ {r}")
        assert_bitwise(_host(p[r:r + 16]), wp, f"codes @ {r}")
        wd = oracle.dequantize(wp, ws, 16, K, global_amax=wA, scale_mode="row", bound=256.0)
        assert_bitwise(_host(xh[r:r + 16]), wd, f"dequantized @ {r}")


def test_max_size_four_over_six_generic_fp32():
    """fp32 rows longer than the row kernel takes (generic kernel), per-row amax
    computed in the pass, MSE."""
    M, K = N_ELEMS // 32768, 32768
    _need_free(48)
    x = _rows_input(M, K, 8, dtype=torch.float32)
    p, s, Ar = nv.quantize_4over6(x, err_mode="mse", e4m3_scale_bound=448, row_scaled=True)
    torch.cuda.synchronize()
    for r in _strips(M, K, 9, n_random=2):
        xs = _host(x[r:r + 16])
        wA = oracle.amax(xs, mode="row")
        assert_bitwise(_host(Ar[r:r + 16]), wA, f"row amax @ {r}")
        wp, ws = oracle.quantize_4over6(xs, wA, err_mode="mse", bound=448.0)
        assert_bitwise(_host(s[r:r + 16]), ws, f"scales @ {r}")
        assert_bitwise(_host(p[r:r + 16]), wp, f"codes @ {r}")


def test_max_size_2d_sr_columnwise_and_tile_dequantize_bf16():
    M, K = N_ELEMS // 8192, 8192
    _need_free(56)
    x = _rows_input(M, K, 10)
    _plant(x)
    A = nv.amax(x)
    assert float(A.item()) == PLANT
    pr, pc, ts = nv.quantize_2d(x, global_amax=A, stochastic=True, seed=SEED, step=STEP,
                                truncation_free=True)
    xh = nv.dequantize(pr, ts, M, K, tile16=True, global_amax=A, bound=448.0)
    torch.cuda.synchronize()
    Ah = np.float32(PLANT)
    for r in _strips(M, K, 11):
        xs = _host(x[r:r + 16])
        wr, wc, wt = oracle.quantize_2d(xs, stochastic=True, seed=SEED, step=STEP, global_amax=Ah,
                                        row_offset=r, truncation_free=True)
        assert_bitwise(_host(ts[r // 16:r // 16 + 1]), wt, f"tile scales @ {r}")
        assert_bitwise(_host(pr[r:r + 16]), wr, f"row codes @ {r}")
        assert_bitwise(_host(pc[:, r // 2:r // 2 + 8]), wc, f"column codes @ {r}")
        wd = oracle.dequantize(wr, wt, 16, K, tile16=True, global_amax=Ah, scale_mode="tensor",
                               bound=448.0)
        assert_bitwise(_host(xh[r:r + 16]), wd, f"dequantized @ {r}")


@pytest.mark.parametrize("fos", [False, True], ids=["standard", "four_over_six"])
def test_max_size_rowcol_bf16(fos):
    M, K = N_ELEMS // 8192, 8192
    _need_free(48)
    x = _rows_input(M, K, 12)
    _plant(x)
    bound = 256.0 if fos else 448.0
    pr, sr, pc, sc = nv.quantize_rowcol(x, "compute", four_over_six=fos, err_mode="mae",
                                        e4m3_scale_bound=bound)
    torch.cuda.synchronize()
    for r in _strips(M, K, 13, n_random=3):
        xs = _host(x[r:r + 16])
        wpr, wsr, wpc, wsc = oracle.quantize_rowcol(xs, np.float32(PLANT), four_over_six=fos,
                                                    err_mode="mae", bound=bound)
        assert_bitwise(_host(sr[r:r + 16]), wsr, f"row scales @ {r}")
        assert_bitwise(_host(pr[r:r + 16]), wpr, f"row codes @ {r}")
        assert_bitwise(_host(sc[:, r // 16:r // 16 + 1]), wsc, f"column scales @ {r}")
        assert_bitwise(_host(pc[:, r // 2:r // 2 + 8]), wpc, f"column codes @ {r}")


def test_max_size_four_over_six_tiles_bf16():
    M, K = N_ELEMS // 8192, 8192
    _need_free(40)
    x = _rows_input(M, K, 14)
    _plant(x)
    pr, pc, ts = nv.quantize_4over6_2d(x, "compute", err_mode="mae", e4m3_scale_bound=256)
    torch.cuda.synchronize()
    for r in _strips(M, K, 15, n_random=3):
        xs = _host(x[r:r + 16])
        wr, wc, wt = oracle.quantize_4over6_2d(xs, np.float32(PLANT), err_mode="mae", bound=256.0)
        assert_bitwise(_host(ts[r // 16:r // 16 + 1]), wt, f"tile scales @ {r}")
        assert_bitwise(_host(pr[r:r + 16]), wr, f"row codes @ {r}")
        assert_bitwise(_host(pc[:, r // 2:r // 2 + 8]), wc, f"column codes @ {r}")
