"""GPU vs CPU-oracle parity (bitwise) for the fused rowwise + columnwise 1x16
quantization and for four-over-six on 16x16 tiles with rowwise and
columnwise outputs, through the C ABI.

Shapes span several workgroups along both axes (a row + column workgroup
covers 256 columns and 256 rows, a 16x16 four-over-six workgroup 512 columns
and 256 rows), ragged row and column tails, grids padded for the XCD work
order, and single-tile tensors."""
import numpy as np
import pytest
import torch

import oracle
import fp4_block_quantization_nvfp4_amd as nv
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np, wide_input
from tests.test_gpu_parity import _specials

pytestmark = pytest.mark.gpu

SHAPES = [(16, 16), (64, 96), (304, 304), (128, 4112), (272, 1040), (48, 512), (528, 784)]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _ga(A):
    return torch.tensor([A], dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("variant", ["std", "fos256-mae", "fos256-mse", "fos448-mae"])
def test_rowcol(shape, bf16, variant):
    M, K = shape
    x = wide_input(M * 7 + K, M, K, bf16, lo=-6, hi=6)
    A = oracle.amax(x)
    fos = variant != "std"
    bound = 448.0 if variant in ("std", "fos448-mae") else 256.0
    err = "mse" if variant.endswith("mse") else "mae"
    wpr, wsr, wpc, wsc = oracle.quantize_rowcol(x, A, four_over_six=fos, err_mode=err, bound=bound)
    pr, sr, pc, sc = nv.quantize_rowcol(to_dev(x), _ga(A), four_over_six=fos, err_mode=err,
                                        e4m3_scale_bound=bound)
    assert_bitwise(to_np(sr), wsr, "row scales")
    assert_bitwise(to_np(pr), wpr, "row codes")
    assert_bitwise(to_np(sc), wsc, "col scales")
    assert_bitwise(to_np(pc), wpc, "col codes")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("err", ["mae", "mse"])
@pytest.mark.parametrize("bound", [256.0, 448.0])
def test_4over6_2d(shape, bf16, err, bound):
    M, K = shape
    x = wide_input(M * 3 + K + 1, M, K, bf16, lo=-6, hi=6)
    A = oracle.amax(x)
    wpr, wpc, wts = oracle.quantize_4over6_2d(x, A, err_mode=err, bound=bound)
    pr, pc, ts = nv.quantize_4over6_2d(to_dev(x), _ga(A), err_mode=err, e4m3_scale_bound=bound)
    assert_bitwise(to_np(ts), wts, "tile scales")
    assert_bitwise(to_np(pr), wpr, "row codes")
    assert_bitwise(to_np(pc), wpc, "col codes")
    pr2, pc2, ts2 = nv.quantize_4over6_2d(to_dev(x), _ga(A), err_mode=err, e4m3_scale_bound=bound,
                                          columnwise=False)
    assert pc2 is None
    assert_bitwise(to_np(pr2), wpr, "row codes (no col)")
    assert_bitwise(to_np(ts2), wts, "tile scales (no col)")
    want = oracle.dequantize(wpr, wts, M, K, tile16=True, global_amax=A, scale_mode="tensor",
                             bound=bound, out="f32")
    got = nv.dequantize(pr, ts, M, K, tile16=True, global_amax=_ga(A), bound=bound,
                        out_dtype=torch.float32)
    assert_bitwise(to_np(got), want, "tile dequant")


def _mixed_tiles():
    """Gaussian tiles, and every other tile column made of values on the
    map-to-4 grid (amax times 1, .75, .5, .375, .25, .125 or 0), which map-to-4
    represents exactly and map-to-6 does not, so both candidates win tiles."""
    import workloads
    x = oracle.bf16_bits_to_f32(wide_input(11, 256, 512, True, lo=-2, hi=2)).copy()
    rng = np.random.default_rng(12)
    lv = np.array([1, 0.75, 0.5, 0.375, 0.25, 0.125, 0], np.float32)
    t = x.reshape(16, 16, 32, 16)
    for i in range(16):
        for j in range(0, 32, 2):
            s = np.float32(2.0 ** rng.integers(-3, 4))
            t[i, :, j, :] = rng.choice(lv, (16, 16)) * s * rng.choice(np.array([-1, 1], np.float32), (16, 16))
            t[i, 0, j, 0] = s
    return workloads.bf16_bits(x)


@pytest.mark.parametrize("shape", [(8192, 7168), (32768, 2048), (8192, 16384)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_4over6_2d_rowwise_strip_counts(shape):
    """Rowwise only, the 16x16 kernel walks 4, 8 or 16 strips per workgroup
    depending on the grid (8192x7168: 4, 32768x2048: 8, 8192x16384: 16); its
    codes and tile scales equal those of the columnwise launch (16 strips)
    everywhere, and the oracle's on the first and last strips."""
    M, K = shape
    x = wide_input(M + K, M, K, True, lo=-6, hi=6)
    A = oracle.amax(x)
    xd = to_dev(x)
    pr, pc, ts = nv.quantize_4over6_2d(xd, _ga(A), err_mode="mae")
    pr2, pc2, ts2 = nv.quantize_4over6_2d(xd, _ga(A), err_mode="mae", columnwise=False)
    assert pc2 is None
    assert torch.equal(pr, pr2) and torch.equal(ts, ts2)
    for rows in (slice(0, 16), slice(M - 16, M)):
        wpr, _, wts = oracle.quantize_4over6_2d(x[rows], A, err_mode="mae")
        assert_bitwise(to_np(pr2[rows]), wpr, "row codes")
        assert_bitwise(to_np(ts2[rows.start // 16:rows.stop // 16]), wts, "tile scales")


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_4over6_2d_picks_both_candidates(err):
    x = _mixed_tiles()
    A = oracle.amax(x)
    wpr, wpc, wts = oracle.quantize_4over6_2d(x, A, err_mode=err)
    a = oracle.nvfp4._nan_drop_absmax(oracle.bf16_bits_to_f32(x).reshape(16, 16, 32, 16), axis=(1, 3))
    S_enc = oracle.nvfp4.global_scales(A, 256.0)[0]
    k6 = oracle.e4m3_encode(np.fmin((a / np.float32(6)) * S_enc, np.float32(448)))
    assert (wts == k6).sum() > 100 and (wts != k6).sum() > 100
    pr, pc, ts = nv.quantize_4over6_2d(to_dev(x), _ga(A), err_mode=err)
    assert_bitwise(to_np(ts), wts)
    assert_bitwise(to_np(pr), wpr)
    assert_bitwise(to_np(pc), wpc)


@pytest.mark.parametrize("bf16", [False, True])
def test_specials_rowcol_and_4over6_2d(bf16):
    x = _specials(bf16)
    xd = to_dev(x)
    for A in (oracle.amax(x), np.float32(3000.0), np.float32(0.0)):
        for fos, bound in ((False, 448.0), (True, 256.0)):
            for err in ("mae", "mse"):
                want = oracle.quantize_rowcol(x, A, four_over_six=fos, err_mode=err, bound=bound)
                got = nv.quantize_rowcol(xd, _ga(A), four_over_six=fos, err_mode=err,
                                         e4m3_scale_bound=bound)
                for g, w, what in zip(got, want, ("pr", "sr", "pc", "sc")):
                    assert_bitwise(to_np(g), w, f"rowcol {what} A={A} fos={fos} {err}")
        for err in ("mae", "mse"):
            wpr, wpc, wts = oracle.quantize_4over6_2d(x, A, err_mode=err)
            pr, pc, ts = nv.quantize_4over6_2d(xd, _ga(A), err_mode=err)
            assert_bitwise(to_np(ts), wts, f"2d scales A={A} {err}")
            assert_bitwise(to_np(pr), wpr, f"2d rows A={A} {err}")
            assert_bitwise(to_np(pc), wpc, f"2d cols A={A} {err}")


def test_rowcol_standard_matches_quantize_and_transpose():
    x = wide_input(21, 160, 272, True, lo=-5, hi=5)
    A = _ga(oracle.amax(x))
    pr, sr, pc, sc = nv.quantize_rowcol(to_dev(x), A)
    p, s = nv.quantize(to_dev(x), global_amax=A)
    assert_bitwise(to_np(pr), to_np(p))
    assert_bitwise(to_np(sr), to_np(s))
    pt, st = nv.quantize(to_dev(np.ascontiguousarray(x.T)), global_amax=A)
    assert_bitwise(to_np(pc), to_np(pt))
    assert_bitwise(to_np(sc), to_np(st))


def test_empty_next():
    x = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    pr, sr, pc, sc = nv.quantize_rowcol(x, 1.0)
    assert pr.shape == (0, 16) and pc.shape == (32, 0) and sc.shape == (32, 0)
    pr, pc, ts = nv.quantize_4over6_2d(x, 1.0)
    assert ts.shape == (0, 2)


def lattice_input(seed, M, K, bf16=True):
    """Blocks whose values sit on small lattices (block scale 2^e * {1, 1.5}
    times k/16, k = 0..16, random signs), plus constant and all-zero blocks:
    both four-over-six candidates often represent such blocks equally well,
    so exact error ties and near ties are common (the cases a choice made
    from approximate error sums must hand to the exact computation)."""
    rng = np.random.default_rng(seed)
    nb = K // 16
    scale = (2.0 ** rng.integers(-6, 7, (M, nb)) * rng.choice([1.0, 1.5, 1.25], (M, nb))).astype(np.float32)
    k = rng.integers(0, 17, (M, nb, 16)).astype(np.float32) / np.float32(16)
    sgn = rng.choice(np.array([-1, 1], np.float32), (M, nb, 16))
    x = (scale[..., None] * k * sgn).astype(np.float32)
    kind = rng.random((M, nb))
    x[kind < 0.05] = 0.0
    const = (kind >= 0.05) & (kind < 0.1)
    x[const] = scale[const][:, None]
    x = x.reshape(M, K)
    if bf16:
        import workloads
        return workloads.bf16_bits(x)
    return x


@pytest.mark.parametrize("shape", [(64, 7168), (48, 512)])
@pytest.mark.parametrize("err", ["mae", "mse"])
@pytest.mark.parametrize("bound", [256.0, 448.0])
def test_four_over_six_ties(shape, err, bound):
    M, K = shape
    x = lattice_input(M + K, M, K)
    xd = to_dev(x)
    # row-scaled, amax computed in the kernel
    Ar = oracle.amax(x, mode="row")
    wp, ws = oracle.quantize_4over6(x, Ar, err_mode=err, bound=bound)
    p, s, ga = nv.quantize_4over6(xd, None, err_mode=err, e4m3_scale_bound=bound, row_scaled=True)
    assert_bitwise(to_np(ga), Ar, "row amax")
    assert_bitwise(to_np(s), ws, "row-scaled scales")
    assert_bitwise(to_np(p), wp, "row-scaled codes")
    # per-tensor amax, and a given amax below the true one (scales clip at 448)
    for A in (oracle.amax(x), np.float32(oracle.amax(x) / 64)):
        wp, ws = oracle.quantize_4over6(x, A, err_mode=err, bound=bound)
        p, s, _ = nv.quantize_4over6(xd, _ga(A), err_mode=err, e4m3_scale_bound=bound, row_scaled=False)
        assert_bitwise(to_np(s), ws, f"tensor scales A={A}")
        assert_bitwise(to_np(p), wp, f"tensor codes A={A}")
        wpr, wsr, wpc, wsc = oracle.quantize_rowcol(x, A, four_over_six=True, err_mode=err, bound=bound)
        got = nv.quantize_rowcol(xd, _ga(A), four_over_six=True, err_mode=err, e4m3_scale_bound=bound)
        for g, w, what in zip(got, (wpr, wsr, wpc, wsc), ("pr", "sr", "pc", "sc")):
            assert_bitwise(to_np(g), w, f"rowcol {what} A={A}")
        wr, wc, wt = oracle.quantize_4over6_2d(x, A, err_mode=err, bound=bound)
        r, c, t = nv.quantize_4over6_2d(xd, _ga(A), err_mode=err, e4m3_scale_bound=bound)
        assert_bitwise(to_np(t), wt, f"2d tiles A={A}")
        assert_bitwise(to_np(r), wr, f"2d rows A={A}")
        assert_bitwise(to_np(c), wc, f"2d cols A={A}")


def identical_dequant_input(seed, M, K, A=3.0, broken=0.0):
    """Blocks whose map-to-6 and map-to-4 candidates dequantize every element
    to the same value, so their error sums tie exactly (zero error for the
    on-grid values, nonzero for the off-grid ones).  Every block holds +-A
    (so a = A, sigma6 = 256 and sigma4 = 384 at bound 256), the rest of its
    elements are A times one of {1, 0.52, 0.5, 0.27, 0.25, 0.02, 0}: map-to-6
    codes 6, 3, 3, 1.5, 1.5, 0, 0 and map-to-4 codes 4, 2, 2, 1, 1, 0, 0.  A
    fraction `broken` of the 16x16 tiles get one element at 0.125 A (map-to-6
    code 1 with error A / 24, map-to-4 code 0.5 with none), which breaks the
    identity and makes map-to-4 win that block and tile."""
    rng = np.random.default_rng(seed)
    lv = np.array([1, 0.52, 0.5, 0.27, 0.25, 0.02, 0], np.float32)
    x = rng.choice(lv, (M, K)) * rng.choice(np.array([-1, 1], np.float32), (M, K))
    x[:, ::16] = rng.choice(np.array([-1, 1], np.float32), (M, K // 16))
    t = x.reshape(M // 16, 16, K // 16, 16)
    hit = rng.random((M // 16, K // 16)) < broken
    t[:, 5, :, 7][hit] = np.float32(0.125)
    import workloads
    return workloads.bf16_bits((x * np.float32(A)).astype(np.float32))


@pytest.mark.parametrize("err", ["mae", "mse"])
@pytest.mark.parametrize("broken", [0.0, 0.3])
@pytest.mark.parametrize("A0", [3.0, 0.0137, 1000.0])
def test_four_over_six_identical_dequant_ties(err, broken, A0):
    M, K = 96, 1040
    x = identical_dequant_input(7 + int(broken * 10), M, K, A=A0, broken=broken)
    xd = to_dev(x)
    A = oracle.amax(x)
    k6 = oracle.e4m3_encode(np.float32(256.0))
    wp, ws = oracle.quantize_4over6(x, A, err_mode=err, bound=256.0)
    # the tie rule keeps map-to-6 wherever the identity holds
    assert (ws == k6).mean() > (0.99 if broken == 0.0 else 0.5)
    assert (ws != k6).any() == (broken > 0)
    p, s, _ = nv.quantize_4over6(xd, _ga(A), err_mode=err, e4m3_scale_bound=256, row_scaled=False)
    assert_bitwise(to_np(s), ws, "1x16 scales")
    assert_bitwise(to_np(p), wp, "1x16 codes")
    want = oracle.quantize_rowcol(x, A, four_over_six=True, err_mode=err, bound=256.0)
    got = nv.quantize_rowcol(xd, _ga(A), four_over_six=True, err_mode=err, e4m3_scale_bound=256)
    for g, w, what in zip(got, want, ("pr", "sr", "pc", "sc")):
        assert_bitwise(to_np(g), w, f"rowcol {what}")
    wr, wc, wt = oracle.quantize_4over6_2d(x, A, err_mode=err, bound=256.0)
    assert (wt == k6).mean() > (0.99 if broken == 0.0 else 0.3)
    assert (wt != k6).any() == (broken > 0)
    r, c, t = nv.quantize_4over6_2d(xd, _ga(A), err_mode=err, e4m3_scale_bound=256)
    assert_bitwise(to_np(t), wt, "2d tiles")
    assert_bitwise(to_np(r), wr, "2d rows")
    assert_bitwise(to_np(c), wc, "2d cols")
