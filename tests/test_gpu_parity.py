"""GPU vs CPU-oracle parity through the C ABI (bitwise: tolerance 0 for
codes, scale bytes, residuals, amaxes and dequantized values).

Shapes span several workgroups and ragged tails (K not a multiple of the
wave's span, M not a multiple of the workgroup's rows), following the shape
lists of the four-over-six pull request's validation (128x128, 256x512,
2048x1024, 304x304, 128x320, 64x1024 ...), scaled to what the oracle finishes
in seconds.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import fp4_block_quantization_nvfp4_amd as nv
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np, wide_input

pytestmark = pytest.mark.gpu

SHAPES = [(1, 16), (3, 48), (128, 128), (304, 304), (128, 320), (257, 4112), (64, 1024)]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("stochastic", [False, True])
@pytest.mark.parametrize("global_scale", [False, True])
def test_quantize_dequantize(shape, bf16, stochastic, global_scale):
    M, K = shape
    x = wide_input(11 + M + K, M, K, bf16)
    A = oracle.amax(x) if global_scale else None
    want_p, want_s = oracle.quantize(x, stochastic=stochastic, seed=3, step=7, global_amax=A)
    xd = to_dev(x)
    ga = torch.tensor([A], device="cuda") if global_scale else None
    p, s = nv.quantize(xd, stochastic=stochastic, seed=3, step=7, global_amax=ga)
    assert_bitwise(to_np(p), want_p, "packed")
    assert_bitwise(to_np(s), want_s, "scales")
    for out_dtype, name in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        want = oracle.dequantize(want_p, want_s, M, K, global_amax=A,
                                 scale_mode="tensor" if global_scale else "none", out=name)
        got = nv.dequantize(p, s, M, K, global_amax=ga, out_dtype=out_dtype)
        assert_bitwise(to_np(got), want, f"dequant {name}")


@pytest.mark.parametrize("shape", [(3, 48), (304, 304), (257, 4112)])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("stochastic", [False, True])
@pytest.mark.parametrize("global_scale", [False, True])
def test_qdq_error_feedback(shape, bf16, stochastic, global_scale):
    M, K = shape
    x = wide_input(5 + M, M, K, bf16)
    r0 = (np.random.default_rng(M + K).standard_normal((M, K)) * 1e-2).astype(np.float32)
    A = oracle.amax(x, r0) if global_scale else None
    r_or = r0.copy()
    want_o, want_p, want_s = oracle.qdq(x, stochastic=stochastic, residual=r_or, seed=1, step=2,
                                        global_amax=A, out="bf16")
    r = to_dev(r0)
    ga = torch.tensor([A], device="cuda") if global_scale else None
    o, p, s = nv.qdq(to_dev(x), stochastic=stochastic, residual=r, seed=1, step=2,
                     global_amax=ga, return_codes=True)
    assert_bitwise(to_np(o), want_o, "qdq out")
    assert_bitwise(to_np(p), want_p, "packed")
    assert_bitwise(to_np(s), want_s, "scales")
    assert_bitwise(to_np(r), r_or, "residual")
    # quantize with residual updates it the same way
    r2 = to_dev(r0)
    p2, s2 = nv.quantize(to_dev(x), stochastic=stochastic, residual=r2, seed=1, step=2, global_amax=ga)
    assert_bitwise(to_np(p2), want_p, "quantize+EF packed")
    assert_bitwise(to_np(r2), r_or, "quantize+EF residual")
    # fp32 output
    r3 = to_dev(r0)
    o3 = nv.qdq(to_dev(x), stochastic=stochastic, residual=r3, seed=1, step=2, global_amax=ga,
                out_dtype=torch.float32)
    want_f = oracle.qdq(x, stochastic=stochastic, residual=r0.copy(), seed=1, step=2,
                        global_amax=A, out="f32")[0]
    assert_bitwise(to_np(o3), want_f, "qdq f32 out")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("where", ["first", "last", "middle", "second_unroll_slot", "tail"])
def test_amax_tensor_positions(bf16, where):
    """Per-tensor amax over 1024x1040 (about 0.5 M 16-byte chunks: every lane
    takes several four-chunk steps and a remainder): the largest magnitude
    planted at one position, NaNs of both signs and an infinity-free rest."""
    M, K = 1024, 1040
    rng = np.random.default_rng(11 if bf16 else 12)
    x = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    flat = x.reshape(-1)
    n = flat.size
    pos = {"first": 0, "last": n - 1, "middle": n // 2 + 3, "second_unroll_slot": 524288 + 9,
           "tail": n - 8 * 1000 - 5}[where]
    flat[pos] = -37.75
    for k in (1, 5000, n // 3, n - 2):
        if k != pos:
            flat[k] = np.float32(np.nan) if k % 2 else -np.float32(np.nan)
    xi = workloads.bf16_bits(x) if bf16 else x
    assert_bitwise(to_np(nv.amax(to_dev(xi), None, "tensor")), np.array([oracle.amax(xi)], np.float32))


@pytest.mark.parametrize("shape", [(1, 16), (128, 320), (257, 4112), (2, 16384)])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("residual", [False, True])
def test_amax(shape, bf16, residual):
    M, K = shape
    x = wide_input(M * 7 + K, M, K, bf16)
    r0 = (np.random.default_rng(1).standard_normal((M, K)) * 1e3).astype(np.float32) if residual else None
    rd = to_dev(r0) if residual else None
    assert_bitwise(to_np(nv.amax(to_dev(x), rd, "tensor")), np.array([oracle.amax(x, r0)], np.float32))
    assert_bitwise(to_np(nv.amax(to_dev(x), rd, "row")), oracle.amax(x, r0, mode="row"))


@pytest.mark.parametrize("shape", [(1, 16), (128, 128), (304, 304), (128, 320), (64, 1024), (33, 7168),
                                   (5, 12288), (3, 16384), (2, 16400)])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("err_mode", ["mae", "mse"])
@pytest.mark.parametrize("bound", [256, 448])
@pytest.mark.parametrize("mode", ["tensor", "row_given", "row_computed"])
def test_four_over_six(shape, bf16, err_mode, bound, mode):
    M, K = shape
    x = wide_input(M + 3 * K, M, K, bf16, lo=-6, hi=6)
    xd = to_dev(x)
    if mode == "tensor":
        A = oracle.amax(x)
        ga = torch.tensor([A], device="cuda")
        p, s, _ = nv.quantize_4over6(xd, ga, err_mode=err_mode, e4m3_scale_bound=bound, row_scaled=False)
    else:
        A = oracle.amax(x, mode="row")
        if mode == "row_given":
            p, s, _ = nv.quantize_4over6(xd, to_dev(A), err_mode=err_mode, e4m3_scale_bound=bound,
                                         row_scaled=True)
        else:
            p, s, ga = nv.quantize_4over6(xd, None, err_mode=err_mode, e4m3_scale_bound=bound,
                                          row_scaled=True)
            assert_bitwise(to_np(ga), A, "row amax")
    want_p, want_s = oracle.quantize_4over6(x, A, err_mode=err_mode, bound=bound)
    assert_bitwise(to_np(s), want_s, "scales")
    assert_bitwise(to_np(p), want_p, "packed")


@pytest.mark.parametrize("shape", [(16, 16), (64, 96), (304, 304), (128, 4112), (32, 512)])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("stochastic", [False, True])
@pytest.mark.parametrize("global_scale", [False, True])
@pytest.mark.parametrize("tf", [False, True], ids=["nearest", "truncfree"])
def test_quantize_2d(shape, bf16, stochastic, global_scale, tf):
    M, K = shape
    x = wide_input(M * 5 + K, M, K, bf16, lo=-8, hi=8)
    A = oracle.amax(x) if global_scale else None
    wr, wc, ws = oracle.quantize_2d(x, stochastic=stochastic, seed=4, step=9, global_amax=A,
                                    truncation_free=tf)
    ga = torch.tensor([A], device="cuda") if global_scale else None
    r, c, s = nv.quantize_2d(to_dev(x), ga, stochastic=stochastic, seed=4, step=9, truncation_free=tf)
    assert_bitwise(to_np(s), ws, "tile scales")
    assert_bitwise(to_np(r), wr, "rowwise")
    assert_bitwise(to_np(c), wc, "columnwise")
    r2, c2, s2 = nv.quantize_2d(to_dev(x), ga, stochastic=stochastic, seed=4, step=9, columnwise=False,
                                truncation_free=tf)
    assert c2 is None
    assert_bitwise(to_np(r2), wr, "rowwise (no col)")
    want = oracle.dequantize(wr, ws, M, K, tile16=True, global_amax=A,
                             scale_mode="tensor" if global_scale else "none", out="f32")
    got = nv.dequantize(r, s, M, K, tile16=True, global_amax=ga, out_dtype=torch.float32)
    assert_bitwise(to_np(got), want, "tile dequant")


@pytest.mark.parametrize("shape", [(48, 528), (80, 1040), (272, 16), (528, 48), (544, 1552)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("stochastic", [False, True], ids=["rtn", "sr"])
def test_quantize_2d_strip_groups(shape, stochastic):
    """Strip counts that leave a lone strip or a partial group at the end of
    a workgroup (3, 5, 17, 33, 34 strips of 16 rows) and ragged last column
    groups (a column group covers 512 columns), bf16 with a per-tensor amax."""
    M, K = shape
    x = wide_input(M * 7 + K, M, K, True, lo=-6, hi=6)
    A = oracle.amax(x)
    wr, wc, ws = oracle.quantize_2d(x, stochastic=stochastic, seed=21, step=3, global_amax=A)
    r, c, s = nv.quantize_2d(to_dev(x), torch.tensor([A], device="cuda"), stochastic=stochastic, seed=21, step=3)
    assert_bitwise(to_np(s), ws, "tile scales")
    assert_bitwise(to_np(r), wr, "rowwise")
    assert_bitwise(to_np(c), wc, "columnwise")


def test_2d_transposition_invariance_on_gpu():
    x = wide_input(99, 64, 128, True, lo=-4, hi=4)
    xt = np.ascontiguousarray(x.T)
    A = torch.tensor([oracle.amax(x)], device="cuda")
    r, c, s = nv.quantize_2d(to_dev(x), A)
    rt, ct, st = nv.quantize_2d(to_dev(xt), A)
    assert_bitwise(to_np(st), to_np(s).T)
    assert_bitwise(to_np(c), to_np(rt))
    assert_bitwise(to_np(ct), to_np(r))


def _specials(bf16):
    M, K = 16, 64
    x = wide_input(7, M, K, False, lo=-3, hi=3)
    x[0, 3] = np.nan
    x[0, 16:32] = np.nan                      # all-NaN block
    x[1, 0:3] = [np.inf, -np.inf, 1.0]
    x[2, :16] = 2.0 ** -140                   # subnormal block
    x[2, 16:32] = np.linspace(-2.0 ** -9.5, 2.0 ** -9.5, 16)
    x[3, :16] = 447.0 * 6
    x[3, 16] = 448.0 * 6 * 1.0001             # near-448 block scale
    x[4, :] = 0.0                             # all-zero row
    x[5, :] = np.float32(2.0) ** np.linspace(-20, 20, K).astype(np.float32)
    x[6, :] = -0.0
    if bf16:
        import workloads
        return workloads.bf16_bits(x)
    return x


@pytest.mark.parametrize("bf16", [False, True])
def test_special_values(bf16):
    x = _specials(bf16)
    M, K = x.shape
    xd = to_dev(x)
    for st in (False, True):
        wp, ws = oracle.quantize(x, stochastic=st, seed=5)
        p, s = nv.quantize(xd, stochastic=st, seed=5)
        assert_bitwise(to_np(p), wp, f"packed sr={st}")
        assert_bitwise(to_np(s), ws, f"scales sr={st}")
        out = nv.qdq(xd, stochastic=st, seed=5, out_dtype=torch.bfloat16)
        assert_bitwise(to_np(out), oracle.qdq(x, stochastic=st, seed=5)[0], "qdq")
    # 2D with a global amax of inf (x has an inf) and without
    for ga_on in (False, True):
        for tf in (False, True):
            A = oracle.amax(x) if ga_on else None
            wr, wc, wts = oracle.quantize_2d(x, global_amax=A, truncation_free=tf)
            r, c, ts = nv.quantize_2d(xd, torch.tensor([A], device="cuda") if ga_on else None,
                                      truncation_free=tf)
            assert_bitwise(to_np(ts), wts)
            assert_bitwise(to_np(r), wr)
            assert_bitwise(to_np(c), wc)
    # four-over-six: per-row amax with NaN/inf rows, amax == 0 rows
    A = oracle.amax(x, mode="row")
    for err in ("mae", "mse"):
        wp, ws = oracle.quantize_4over6(x, A, err_mode=err)
        p, s, ga = nv.quantize_4over6(xd, None, err_mode=err, row_scaled=True)
        assert_bitwise(to_np(ga), A, "row amax")
        assert_bitwise(to_np(s), ws, "4o6 scales")
        assert_bitwise(to_np(p), wp, "4o6 packed")
        At = oracle.amax(x)  # inf
        wp, ws = oracle.quantize_4over6(x, At, err_mode=err)
        p, s, _ = nv.quantize_4over6(xd, torch.tensor([At], device="cuda"), err_mode=err, row_scaled=False)
        assert_bitwise(to_np(s), ws, "4o6 inf-amax scales")
        assert_bitwise(to_np(p), wp, "4o6 inf-amax packed")


def test_error_feedback_class_and_resume():
    # fp4-train, API ErrorFeedback; the generator is counter-based, so a run
    # split by a save/restore of the residual is bit-identical.
    x0 = to_dev(wide_input(3, 64, 256, True, lo=-2, hi=2))
    ef = nv.ErrorFeedback(stochastic=True, seed=9)
    outs = [ef.qdq("w", x0, step=t) for t in range(10)]
    ef2 = nv.ErrorFeedback(stochastic=True, seed=9)
    for t in range(5):
        ef2.qdq("w", x0, step=t)
    state = ef2.state_dict()
    ef3 = nv.ErrorFeedback(stochastic=True, seed=9)
    ef3.load_state_dict(state)
    outs3 = [ef3.qdq("w", x0, step=t) for t in range(5, 10)]
    for a, b in zip(outs[5:], outs3):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(ef.residuals["w"].view(torch.int32), ef3.residuals["w"].view(torch.int32))


def test_sr_statistics_on_gpu():
    # fp4-train, Correctness: SR mean for 2.3 is 2.300 (RTN 2.000).
    blocks = 1 << 16
    x = np.full((blocks, 16), 2.3, np.float32)
    x[:, 0] = 6.0
    xd = to_dev(x)
    vals = torch.cat([nv.qdq(xd, stochastic=True, seed=0, step=s, out_dtype=torch.float32)[:, 1:].reshape(-1)
                      for s in range(4)]).double()
    assert f"{vals.mean().item():.3f}" == "2.300"
    rtn = nv.qdq(xd, out_dtype=torch.float32)[:, 1:]
    assert f"{rtn.double().mean().item():.3f}" == "2.000"


def test_empty_tensors():
    x = torch.empty((0, 32), device="cuda")
    p, s = nv.quantize(x)
    assert p.shape == (0, 16)
    assert nv.amax(x).item() == 0.0
    x2 = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    r, c, t = nv.quantize_2d(x2)
    assert r.shape == (0, 16)


def _negative_nans(bf16):
    """Finite blocks with NaNs of either sign in them (bf16 0xFFC0 / fp32
    0xFFC00000 is a NaN with the sign bit set), an all-negative-NaN block and
    a NaN next to an infinity.  Every NaN encodes as code 0x7 whatever its
    sign, and the blocks' scales come from their NaN-dropping amaxes."""
    M, K = 32, 128
    x = wide_input(29, M, K, False, lo=-3, hi=3)
    u = x.view(np.uint32)
    neg, pos = np.uint32(0xFFC00000), np.uint32(0x7FC00000)
    u[0, 5] = neg
    u[1, 3] = neg
    u[1, 9] = pos
    u[2, 16:32] = neg
    u[3, 40] = neg
    x[3, 41] = np.inf
    u[5::3, 7::11] = neg
    u[17, 64:80] = neg
    if bf16:
        import workloads
        b = workloads.bf16_bits(x)
        b[np.isnan(x)] = np.where(np.signbit(x[np.isnan(x)]), 0xFFC0, 0x7FC0).astype(np.uint16)
        return b
    return x


@pytest.mark.parametrize("bf16", [False, True])
def test_negative_nan_blocks(bf16):
    x = _negative_nans(bf16)
    xf = oracle.bf16_bits_to_f32(x) if bf16 else x
    assert np.signbit(xf[np.isnan(xf)]).sum() > 10
    M, K = x.shape
    xd = to_dev(x)
    # the tensor holds an infinity: per-tensor paths also run with the largest
    # finite magnitude as amax, so that NaN blocks sit among in-range blocks
    A = np.float32(np.abs(xf[np.isfinite(xf)]).max())
    assert oracle.amax(x) == np.inf
    for st in (False, True):
        wp, ws = oracle.quantize(x, stochastic=st, seed=3)
        p, s = nv.quantize(xd, stochastic=st, seed=3)
        assert_bitwise(to_np(s), ws, f"quantize scales sr={st}")
        assert_bitwise(to_np(p), wp, f"quantize codes sr={st}")
    for err in ("mae", "mse"):
        Ar = oracle.amax(x, mode="row")
        wp, ws = oracle.quantize_4over6(x, Ar, err_mode=err)
        p, s, ga = nv.quantize_4over6(xd, None, err_mode=err, row_scaled=True)
        assert_bitwise(to_np(ga), Ar, f"row amax {err}")
        assert_bitwise(to_np(s), ws, f"4over6 row-computed scales {err}")
        assert_bitwise(to_np(p), wp, f"4over6 row-computed codes {err}")
        p, s, _ = nv.quantize_4over6(xd, torch.from_numpy(Ar).cuda(), err_mode=err)
        assert_bitwise(to_np(s), ws, f"4over6 row-given scales {err}")
        assert_bitwise(to_np(p), wp, f"4over6 row-given codes {err}")
        for At in (A, oracle.amax(x)):
            wp, ws = oracle.quantize_4over6(x, At, err_mode=err)
            p, s, _ = nv.quantize_4over6(xd, torch.tensor([At], device="cuda"), err_mode=err,
                                         row_scaled=False)
            assert_bitwise(to_np(s), ws, f"4over6 tensor scales {err} A={At}")
            assert_bitwise(to_np(p), wp, f"4over6 tensor codes {err} A={At}")
        want = oracle.quantize_rowcol(x, A, four_over_six=True, err_mode=err, bound=256.0)
        got = nv.quantize_rowcol(xd, torch.tensor([A], device="cuda"), four_over_six=True, err_mode=err,
                                 e4m3_scale_bound=256)
        for g, w, what in zip(got, want, ("pr", "sr", "pc", "sc")):
            assert_bitwise(to_np(g), w, f"rowcol fos {what} {err}")
        wr, wc, wt = oracle.quantize_4over6_2d(x, A, err_mode=err)
        r, c, t = nv.quantize_4over6_2d(xd, torch.tensor([A], device="cuda"), err_mode=err)
        assert_bitwise(to_np(t), wt, f"4over6 2d tiles {err}")
        assert_bitwise(to_np(r), wr, f"4over6 2d rows {err}")
        assert_bitwise(to_np(c), wc, f"4over6 2d cols {err}")
    want = oracle.quantize_rowcol(x, A)
    got = nv.quantize_rowcol(xd, torch.tensor([A], device="cuda"))
    for g, w, what in zip(got, want, ("pr", "sr", "pc", "sc")):
        assert_bitwise(to_np(g), w, f"rowcol std {what}")
    for st in (False, True):
        wr, wc, wt = oracle.quantize_2d(x, stochastic=st, seed=1, global_amax=A)
        r, c, t = nv.quantize_2d(xd, torch.tensor([A], device="cuda"), stochastic=st, seed=1)
        assert_bitwise(to_np(t), wt, f"2d tiles sr={st}")
        assert_bitwise(to_np(r), wr, f"2d rows sr={st}")
        assert_bitwise(to_np(c), wc, f"2d cols sr={st}")


@pytest.mark.parametrize("seed,step", [(0xFFFFFFFF, 0xFFFFFFFF), (0x80000000, 0), (0, 0x80000001),
                                       (123456789, 987654321)])
def test_stochastic_rounding_extreme_seeds(seed, step):
    """Seeds and steps at the ends of their 32-bit range key the same draws
    on both sides (1x16 quantize and qdq with error feedback, 2D)."""
    M, K = 48, 272
    for bf16 in (False, True):
        x = wide_input(seed % 1000 + step % 1000, M, K, bf16, lo=-4, hi=4)
        xd = to_dev(x)
        wp, ws = oracle.quantize(x, stochastic=True, seed=seed, step=step)
        p, s = nv.quantize(xd, stochastic=True, seed=seed, step=step)
        assert_bitwise(to_np(s), ws, "scales")
        assert_bitwise(to_np(p), wp, "codes")
        r0 = (np.random.default_rng(3).standard_normal((M, K)) * 1e-3).astype(np.float32)
        r_or = r0.copy()
        wo = oracle.qdq(x, stochastic=True, residual=r_or, seed=seed, step=step)[0]
        r = to_dev(r0)
        o = nv.qdq(xd, stochastic=True, residual=r, seed=seed, step=step)
        assert_bitwise(to_np(o), wo, "qdq out")
        assert_bitwise(to_np(r), r_or, "qdq residual")
        A = oracle.amax(x)
        wr, wc, wt = oracle.quantize_2d(x, stochastic=True, seed=seed, step=step, global_amax=A)
        rr, cc, tt = nv.quantize_2d(xd, torch.tensor([A], device="cuda"), stochastic=True, seed=seed, step=step)
        assert_bitwise(to_np(tt), wt, "2d tiles")
        assert_bitwise(to_np(rr), wr, "2d rows")
        assert_bitwise(to_np(cc), wc, "2d cols")


@pytest.mark.parametrize("K", [2048, 2064, 4096, 6144, 8192, 14336, 16368, 16384])
def test_four_over_six_row_kernel_block_counts(K):
    """The bf16 row kernel holds ceil(K / 2048) blocks per lane: row lengths
    at and just past each multiple of 2048 columns, for every amax mode."""
    M = 5
    x = wide_input(K, M, K, True, lo=-6, hi=6)
    xd = to_dev(x)
    Ar = oracle.amax(x, mode="row")
    for err in ("mae", "mse"):
        wp, ws = oracle.quantize_4over6(x, Ar, err_mode=err)
        p, s, ga = nv.quantize_4over6(xd, None, err_mode=err, row_scaled=True)
        assert_bitwise(to_np(ga), Ar, "row amax")
        assert_bitwise(to_np(s), ws, "row-computed scales")
        assert_bitwise(to_np(p), wp, "row-computed codes")
        p, s, _ = nv.quantize_4over6(xd, torch.from_numpy(Ar).cuda(), err_mode=err)
        assert_bitwise(to_np(s), ws, "row-given scales")
        assert_bitwise(to_np(p), wp, "row-given codes")
        A = oracle.amax(x)
        wp, ws = oracle.quantize_4over6(x, A, err_mode=err)
        p, s, _ = nv.quantize_4over6(xd, torch.tensor([A], device="cuda"), err_mode=err, row_scaled=False)
        assert_bitwise(to_np(s), ws, "tensor scales")
        assert_bitwise(to_np(p), wp, "tensor codes")
