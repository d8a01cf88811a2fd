"""Seeded special-value fuzz: GPU vs CPU oracle, bit for bit, through every
entry point.

Each case is a random tensor (bf16 or fp32) whose elements are sprinkled
with NaNs of either sign, infinities of either sign, fp32 and bf16
subnormals, signed zeros, values near the e4m3 and e2m1 limits and huge
magnitudes, on top of blocks of widely varying scale, plus whole special
blocks and rows.  Every quantizer runs with several second-level amaxes: the
tensor's own (infinite: two rows hold infinities), its largest finite
magnitude, the 90th percentile of the block amaxes, a larger one, zero and,
for 1x16 paths, per-row vectors.  Any
disagreement with the oracle names the entry point, the case and the first
differing element.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import fp4_block_quantization_nvfp4_amd as nv
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

SPECIAL_BITS = np.array([
    0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF812345,   # NaNs (quiet and signalling, both signs)
    0x7F800000, 0xFF800000,                           # +-inf
    0x00000001, 0x80000001, 0x007FFFFF, 0x00400000,   # fp32 subnormals
    0x00000000, 0x80000000,                           # signed zeros
    0x7F7FFFFF, 0xFF7FFFFF, 0x7F000000,               # huge
    0x00800000, 0x02000000, 0x0C000000,               # tiny normals (2^-126, 2^-123, 2^-103)
], np.uint32)
HUGE_BITS = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F000000], np.uint32)
INF_BITS = np.array([0x7F800000, 0xFF800000], np.uint32)
SPECIAL_VALUES = np.array([448.0, -448.0, 2688.0, 6.0, -6.0, 5.0, 0.25, 0.75, 2.0 ** -9,
                           2.0 ** -10, 1.5 * 2.0 ** -9], np.float32)


def fuzz_input(seed, M, K, bf16, wide=False, p_special=0.01):
    """wide: block scales e^-30 .. e^30 and the huge specials; otherwise
    block scales e^-8 .. e^8 and no value near FLT_MAX, so that most blocks
    sit well inside the range of the tensor's amax."""
    rng = np.random.default_rng(seed)
    span = 30.0 if wide else 8.0
    scale = np.exp(rng.uniform(-span, span, (M, K // 16))).repeat(16, axis=1).astype(np.float32)
    x = (rng.standard_normal((M, K)).astype(np.float32) * scale).astype(np.float32)
    u = x.view(np.uint32)
    hit = rng.random((M, K)) < p_special
    pool = SPECIAL_BITS[~np.isin(SPECIAL_BITS, INF_BITS if wide else np.concatenate([INF_BITS, HUGE_BITS]))]
    u[hit] = rng.choice(pool, hit.sum())
    # infinities in two rows only, so that most rows keep a finite amax
    for r in (1 % M, M // 2):
        u[r, rng.choice(K, 2, replace=False)] = rng.choice(INF_BITS, 2)
    hit2 = rng.random((M, K)) < p_special
    x[hit2] = rng.choice(SPECIAL_VALUES, hit2.sum()) * rng.choice(np.array([1.0, 1e-3, 1e-6], np.float32),
                                                                   hit2.sum())
    nb = M * K // 16
    blocks = x.reshape(nb, 16)
    for b in rng.choice(nb, min(nb, 6), replace=False):
        kind = rng.integers(0, 6)
        if kind == 0:
            blocks[b] = 0.0
        elif kind == 1:
            blocks[b].view(np.uint32)[:] = rng.choice(SPECIAL_BITS[:4], 16)    # all NaN
        elif kind == 2:
            blocks[b] = -0.0
        elif kind == 3:
            blocks[b].view(np.uint32)[:] = rng.integers(1, 0x00800000, 16).astype(np.uint32)  # subnormal
        elif kind == 4:
            blocks[b] = np.float32(2.0 ** rng.integers(-20, 20)) * rng.choice([-1, 1], 16)   # constant magnitude
        else:
            blocks[b] = rng.choice(SPECIAL_VALUES, 16)
    if bf16:
        b = workloads.bf16_bits(x)
        nan = np.isnan(x)
        # keep each NaN's sign (the bf16 helper canonicalises NaN to positive)
        b[nan] = np.where(np.signbit(x[nan]), 0xFFC1, 0x7FC1).astype(np.uint16)
        return b
    return x


def assert_bitwise_nan_free(got, want, what):
    """Bitwise equality except where both sides are NaN: the residual of a NaN
    element is NaN, and no passage fixes a NaN's payload."""
    g, w = np.asarray(got), np.asarray(want)
    both = np.isnan(g) & np.isnan(w)
    assert_bitwise(np.where(both, np.float32(0), g), np.where(both, np.float32(0), w), what)


def _f32(x):
    return oracle.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def _tensor_amaxes(x):
    """The tensor's amax (infinite here), its largest finite magnitude, the
    90th percentile of the finite block amaxes (blocks on both sides of it),
    a larger amax and zero."""
    xf = _f32(x)
    fin = np.abs(xf[np.isfinite(xf)])
    Af = np.float32(fin.max()) if fin.size else np.float32(0.0)
    a = np.abs(np.where(np.isfinite(xf), xf, 0)).reshape(-1, 16).max(axis=1)
    Ap = np.float32(np.percentile(a, 90))
    with np.errstate(over="ignore"):
        return [oracle.amax(x), Af, Ap, np.float32(Af * 3), np.float32(0.0)]


def _ga(A):
    return torch.tensor([A], dtype=torch.float32, device="cuda")


CASES = [(s, M, K, bf16, wide)
         for s, (M, K) in enumerate([(16, 64), (32, 272), (48, 1040), (64, 512), (96, 2064), (16, 16400)])
         for bf16 in (False, True) for wide in (False, True)]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("seed,M,K,bf16,wide", CASES)
def test_fuzz_1x16_standard(seed, M, K, bf16, wide):
    x = fuzz_input(100 + seed, M, K, bf16, wide)
    xd = to_dev(x)
    for A in [None] + _tensor_amaxes(x):
        for sr in (False, True):
            wp, ws = oracle.quantize(x, stochastic=sr, seed=seed, step=3, global_amax=A)
            p, s = nv.quantize(xd, stochastic=sr, seed=seed, step=3,
                               global_amax=None if A is None else _ga(A))
            assert_bitwise(to_np(s), ws, f"quantize scales A={A} sr={sr}")
            assert_bitwise(to_np(p), wp, f"quantize codes A={A} sr={sr}")
        r0 = fuzz_input(200 + seed, M, K, False, p_special=0.002)
        r0[~np.isfinite(r0)] = 0.0
        r0 *= np.float32(1e-3)
        r_or = r0.copy()
        wo, wp, ws = oracle.qdq(x, stochastic=True, residual=r_or, seed=seed, step=1, global_amax=A)
        r = to_dev(r0)
        o, p, s = nv.qdq(xd, stochastic=True, residual=r, seed=seed, step=1,
                         global_amax=None if A is None else _ga(A), return_codes=True)
        assert_bitwise(to_np(s), ws, f"qdq scales A={A}")
        assert_bitwise(to_np(p), wp, f"qdq codes A={A}")
        assert_bitwise(to_np(o), wo, f"qdq out A={A}")
        assert_bitwise_nan_free(to_np(r), r_or, f"qdq residual A={A}")
        if A is not None:
            want = oracle.dequantize(wp, ws, M, K, global_amax=A, scale_mode="tensor", out="f32")
            got = nv.dequantize(p, s, M, K, global_amax=_ga(A), out_dtype=torch.float32)
            assert_bitwise(to_np(got), want, f"dequantize A={A}")


@pytest.mark.parametrize("seed,M,K,bf16,wide", CASES)
def test_fuzz_amax(seed, M, K, bf16, wide):
    x = fuzz_input(500 + seed, M, K, bf16, wide)
    xd = to_dev(x)
    r0 = fuzz_input(600 + seed, M, K, False, wide)
    for r in (None, r0):
        rd = None if r is None else to_dev(r)
        assert_bitwise(to_np(nv.amax(xd, rd, "tensor")), np.array([oracle.amax(x, r)], np.float32),
                       f"tensor amax res={r is not None}")
        assert_bitwise(to_np(nv.amax(xd, rd, "row")), oracle.amax(x, r, mode="row"),
                       f"row amax res={r is not None}")


@pytest.mark.parametrize("seed,M,K,bf16,wide", CASES)
@pytest.mark.parametrize("err", ["mae", "mse"])
def test_fuzz_four_over_six_1x16(seed, M, K, bf16, wide, err):
    x = fuzz_input(300 + seed, M, K, bf16, wide)
    xd = to_dev(x)
    Ar = oracle.amax(x, mode="row")
    wp, ws = oracle.quantize_4over6(x, Ar, err_mode=err)
    p, s, ga = nv.quantize_4over6(xd, None, err_mode=err, row_scaled=True)
    assert_bitwise(to_np(ga), Ar, "row amax")
    assert_bitwise(to_np(s), ws, "row-computed scales")
    assert_bitwise(to_np(p), wp, "row-computed codes")
    Ag = (Ar * np.float32(0.7)).astype(np.float32)
    wp, ws = oracle.quantize_4over6(x, Ag, err_mode=err, bound=448.0)
    p, s, _ = nv.quantize_4over6(xd, torch.from_numpy(Ag).cuda(), err_mode=err, e4m3_scale_bound=448)
    assert_bitwise(to_np(s), ws, "row-given scales")
    assert_bitwise(to_np(p), wp, "row-given codes")
    for A in _tensor_amaxes(x):
        wp, ws = oracle.quantize_4over6(x, A, err_mode=err)
        p, s, _ = nv.quantize_4over6(xd, _ga(A), err_mode=err, row_scaled=False)
        assert_bitwise(to_np(s), ws, f"tensor scales A={A}")
        assert_bitwise(to_np(p), wp, f"tensor codes A={A}")


@pytest.mark.parametrize("seed,M,K,bf16,wide", CASES)
def test_fuzz_2d_rowcol(seed, M, K, bf16, wide):
    x = fuzz_input(400 + seed, M, K, bf16, wide)
    xd = to_dev(x)
    for A in _tensor_amaxes(x):
        for sr, tf in ((False, False), (True, False), (True, True)):
            wr, wc, wt = oracle.quantize_2d(x, stochastic=sr, seed=seed, step=2, global_amax=A,
                                            truncation_free=tf)
            r, c, t = nv.quantize_2d(xd, _ga(A), stochastic=sr, seed=seed, step=2, truncation_free=tf)
            assert_bitwise(to_np(t), wt, f"2d tiles A={A} sr={sr} tf={tf}")
            assert_bitwise(to_np(r), wr, f"2d rows A={A} sr={sr} tf={tf}")
            assert_bitwise(to_np(c), wc, f"2d cols A={A} sr={sr} tf={tf}")
        for fos, err in ((False, "mae"), (True, "mae"), (True, "mse")):
            bound = 256.0 if fos else 448.0
            want = oracle.quantize_rowcol(x, A, four_over_six=fos, err_mode=err, bound=bound)
            got = nv.quantize_rowcol(xd, _ga(A), four_over_six=fos, err_mode=err, e4m3_scale_bound=bound)
            for g, w, what in zip(got, want, ("pr", "sr", "pc", "sc")):
                assert_bitwise(to_np(g), w, f"rowcol {what} A={A} fos={fos} {err}")
        for err in ("mae", "mse"):
            wr, wc, wt = oracle.quantize_4over6_2d(x, A, err_mode=err)
            r, c, t = nv.quantize_4over6_2d(xd, _ga(A), err_mode=err)
            assert_bitwise(to_np(t), wt, f"4over6 2d tiles A={A} {err}")
            assert_bitwise(to_np(r), wr, f"4over6 2d rows A={A} {err}")
            assert_bitwise(to_np(c), wc, f"4over6 2d cols A={A} {err}")
