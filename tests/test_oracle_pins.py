"""Pins of the oracle against values the pages print, closed forms and
invariants (CPU only).

Cited passages: "fp4-train" card (Method, Correctness, Requirements and
limits); four-over-six pull request (What, CuTe DSL kernel Design, Bitwise
validation); "Stable FP4 Training via Transposition-Invariant Block
Quantization" (abstract).
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle.nvfp4 import code_values, unpack_codes
from tests.test_oracle_formats import page_values

F32 = np.float32
PV = page_values()


def _fmt3(x):
    return f"{x:.3f}"


# ---------------------------------------------------------------- scale rule

def test_block_absmax_six_gives_unit_scale():
    # fp4-train, Method: scale = block_absmax / 6; a = 6 -> sigma = 1 -> 0x38,
    # and on-grid values come back exactly.
    x = np.array([[6.0, 1.5, -3.0, 0.5, -0.0, 4.0, 2.0, 1.0] * 2], F32)
    packed, scales = oracle.quantize(x)
    assert scales.tolist() == [[0x38]]
    out = oracle.dequantize(packed, scales, 1, 16, out="f32")
    assert np.array_equal(out.view(np.uint32), x.view(np.uint32))


def test_constant_block_saturates_at_six():
    # All-2.3 block: sigma = 2.3/6 -> e4m3 0.375; 2.3 * (1/0.375) > 6 saturates,
    # so it dequantizes to 6 * 0.375 = 2.25 (why the 2.3 demo uses unit scale).
    x = np.full((1, 16), 2.3, F32)
    packed, scales = oracle.quantize(x)
    assert oracle.E4M3_VALUES[scales[0, 0]] == F32(0.375)
    out = oracle.dequantize(packed, scales, 1, 16, out="f32")
    assert np.all(out == F32(2.25))


# ------------------------------------------------------------ 2.3 examples

def _unit_scale_block(val, dtype=np.float32):
    x = np.full((1, 16), val, F32)
    x[0, 0] = 6.0
    return x if dtype == np.float32 else workloads.bf16_bits(x)


def test_rtn_of_2p3_is_2():
    # fp4-train, Correctness: round-to-nearest gives 2.000 for 2.3.
    packed, scales = oracle.quantize(_unit_scale_block(2.3))
    codes = unpack_codes(packed)
    assert scales[0, 0] == 0x38 and np.all(codes[0, 1:] == 0x4)
    out = oracle.dequantize(packed, scales, 1, 16, out="f32")
    assert _fmt3(out[0, 1]) == _fmt3(PV["rtn_2p3"][0])


def test_sr_mean_of_2p3():
    # fp4-train, Correctness: the SR mean is 2.300.  Closed form: with
    # f = fl(2.3) - 2 and a 16-bit draw, P(up) = ceil(f * 2**16) / 2**16.
    f = float(F32(2.3) - F32(2.0))
    expect = 2.0 + np.ceil(f * 65536.0) / 65536.0
    assert _fmt3(expect) == _fmt3(PV["sr_mean_2p3"][0])
    blocks = 1 << 17
    x = np.tile(_unit_scale_block(2.3), (blocks, 1))
    vals = []
    for step in range(2):
        out = oracle.qdq(x, stochastic=True, seed=0, step=step, out="f32")[0]
        vals.append(out[:, 1:].reshape(-1))
    v = np.concatenate(vals).astype(np.float64)
    assert set(np.unique(v)) == {2.0, 3.0}
    sd = np.sqrt(0.3 * 0.7 / v.size)
    assert abs(v.mean() - expect) < 5 * sd
    assert _fmt3(v.mean()) == "2.300"


def test_rtn_error_feedback_time_average_of_bf16_2p3():
    # fp4-train, Correctness: RTN plus error feedback time-averages to 2.297.
    # bf16(2.3) = 2.296875 = 2 + 19/64; at unit scale all arithmetic is exact
    # and the residual returns to 0 every 64 steps, so the 64-step mean is
    # exactly 2.296875.
    x = _unit_scale_block(2.3, np.uint16)
    r = np.zeros((1, 16), F32)
    outs = []
    for step in range(64):
        out = oracle.qdq(x, residual=r, step=step, out="f32")[0]
        outs.append(out[0, 1])
    assert r[0, 1] == 0.0
    mean = float(np.mean(np.array(outs, np.float64)))
    assert mean == 2.296875
    assert _fmt3(mean) == _fmt3(PV["rtn_ef_time_average_2p3"][0])
    assert set(outs) == {F32(2.0), F32(3.0)}


def test_rtn_error_feedback_time_average_of_fp32_2p3():
    # Closed form: mean_T = c - (r_T - r_0) / T with |r_T| <= half a grid step.
    x = _unit_scale_block(2.3)
    r = np.zeros((1, 16), F32)
    acc = 0.0
    T = 1000
    for step in range(T):
        acc += float(oracle.qdq(x, residual=r, out="f32")[0][0, 1])
    assert abs(acc / T - float(F32(2.3))) <= 0.5 / T + 1e-12
    assert abs(acc / T - (float(F32(2.3)) - float(r[0, 1]) / T)) < 1e-9


def test_rtn_without_feedback_stalls():
    # fp4-train, intro/Correctness: once the update is below a quantization
    # step, round-to-nearest discards it and the stored weight never moves.
    w = workloads.bf16_bits(_unit_scale_block(1.0))
    w0 = w.copy()
    for step in range(20):
        x = oracle.bf16_bits_to_f32(w) - F32(1e-4)
        w = oracle.qdq(x, step=step)[0]
    assert np.array_equal(w, w0)


# ------------------------------------------------------ EF invariant (C2)

@pytest.mark.parametrize("stochastic", [False, True])
def test_error_feedback_telescopes(stochastic):
    # x_hat_T + r_T = W0 - lr * sum(g_t) up to the fp32 roundings of the two
    # per-step adds (each at most half an ulp of the running value).
    shape, T, lr = (32, 64), 40, F32(1e-4)
    w = workloads.ef_weight0(shape)
    w0 = oracle.bf16_bits_to_f32(w).astype(np.float64)
    r = np.zeros(shape, F32)
    upd = np.zeros(shape, np.float64)
    bound = np.zeros(shape, np.float64)
    for t in range(T):
        g = workloads.ef_grad(t, shape)
        d = g * lr
        x = oracle.bf16_bits_to_f32(w) - d
        upd += d
        out, _, _ = oracle.qdq(x, stochastic=stochastic, residual=r, seed=0, step=t, out="f32")
        # bf16 of the output is exact: val * s has at most 6 significant bits
        w_next = oracle.f32_to_bf16_bits(out)
        assert np.array_equal(oracle.bf16_bits_to_f32(w_next), out)
        w = w_next
        bound += np.spacing(np.abs(x).astype(F32)).astype(np.float64) + \
            np.spacing(np.abs(x + r).astype(F32) + np.abs(out)).astype(np.float64)
    lhs = oracle.bf16_bits_to_f32(w).astype(np.float64) + r
    assert np.all(np.abs(lhs - (w0 - upd)) <= bound)


def test_rtn_qdq_is_idempotent_for_normal_scales():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-3, 3, (64, 1)))).astype(F32)
    y = oracle.qdq(x, out="f32")[0]
    z = oracle.qdq(y, out="f32")[0]
    a = np.abs(x).reshape(64, 16, 16).max(axis=2)
    normal = (a / 6 >= 2.0 ** -6) & (a / 6 <= 448)
    yb, zb = y.reshape(64, 16, 16), z.reshape(64, 16, 16)
    assert normal.mean() > 0.9
    assert np.array_equal(yb[normal], zb[normal])


def test_rtn_error_is_at_most_half_a_grid_step():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 128)) * 3).astype(F32)
    packed, scales = oracle.quantize(x)
    s = np.repeat(oracle.E4M3_VALUES[scales], 16, axis=1)
    q = code_values(unpack_codes(packed))
    v = np.abs(x) / s
    gap = np.select([v < 2, v < 4], [0.5, 1.0], 2.0)
    inside = v <= 6
    err = np.abs(np.abs(x) - np.abs(q) * s)
    assert np.all(err[inside] <= 0.5 * gap[inside] * s[inside] * (1 + 2 ** -20))


# ------------------------------------------------------------ four-over-six

def test_four_over_six_bound_argument():
    # What: bound 256 so that 256 * 1.5 = 384 < 448 (no e4m3 clipping).
    b, e, m = PV["four_over_six_bound"][0], PV["four_over_six_expansion"][0], PV["e4m3_max"][0]
    assert b * e == PV["four_over_six_expanded_scale"][0] < m
    assert oracle.E4M3_VALUES[oracle.e4m3_encode(F32(b * e))] == F32(384.0)


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_four_over_six_tie_picks_map_to_six(err):
    # A = 1536, bound 256: D = 1536, S_enc = S_dec = 1.  Block [1536, 0 x 15]:
    # sigma6 = 256 (0x78), sigma4 = 384 (0x7C); both encodings are exact, the
    # errors tie at 0, so map-to-6 wins: scale 0x78, code 0x7.
    x = np.zeros((1, 16), F32)
    x[0, 0] = 1536.0
    packed, scales = oracle.quantize_4over6(x, F32(1536.0), err_mode=err, bound=256)
    assert scales.tolist() == [[0x78]]
    assert unpack_codes(packed)[0].tolist() == [0x7] + [0] * 15


@pytest.mark.parametrize("err", ["mae", "mse"])
def test_four_over_six_map_to_four_wins(err):
    # Block [1536, 1152, 0 x 14]: map-to-6 gives 1152/256 = 4.5 -> 4 (error
    # 128 MAE / 16384 MSE); map-to-4 gives 1152 * fl(1/384) = 3 exactly
    # (error 0), so scale 0x7C with codes [6, 5, 0, ...].
    x = np.zeros((1, 16), F32)
    x[0, :2] = [1536.0, 1152.0]
    packed, scales = oracle.quantize_4over6(x, F32(1536.0), err_mode=err, bound=256)
    assert scales.tolist() == [[0x7C]]
    assert unpack_codes(packed)[0].tolist() == [0x6, 0x5] + [0] * 14


@pytest.mark.parametrize("block", ["1x16", "16x16"])
def test_four_over_six_scales_never_clip_with_bound_256(block):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-4, 4, (64, 1)))).astype(F32)
    A = oracle.amax(x)
    for err in ("mae", "mse"):
        _, scales = oracle.quantize_4over6(x, A, err_mode=err, bound=256, block=block)
        assert scales.max() <= 0x7C
    _, scales = oracle.quantize_4over6(x, oracle.amax(x, mode="row"), bound=256)
    assert scales.max() <= 0x7C


def test_four_over_six_zero_row():
    x = np.zeros((2, 32), F32)
    x[1] = np.linspace(-1, 1, 32)
    packed, scales = oracle.quantize_4over6(x, oracle.amax(x, mode="row"))
    assert np.all(scales[0] == 0) and np.all(packed[0] == 0)
    assert np.all(scales[1] > 0)


def test_four_over_six_row_variant_equals_per_row_tensor_calls():
    rng = np.random.default_rng(1)
    x = workloads.bf16_bits((rng.standard_normal((8, 64)) * np.exp(rng.uniform(-5, 5, (8, 1)))).astype(F32))
    A = oracle.amax(x, mode="row")
    p, s = oracle.quantize_4over6(x, A, err_mode="mse")
    for m in range(8):
        pm, sm = oracle.quantize_4over6(x[m:m + 1], A[m], err_mode="mse")
        assert np.array_equal(p[m], pm[0]) and np.array_equal(s[m], sm[0])


def test_four_over_six_picks_lower_error_candidate():
    # With A = D (S_enc = S_dec = 1) each block's output must be one of the
    # two candidate encodings, and the kept one must have the lower error
    # (checked in float64 on blocks whose two errors differ clearly).
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((128, 64)) * 20).astype(F32)
    x[0, 0] = 1536.0
    packed, scales = oracle.quantize_4over6(x, F32(1536.0), err_mode="mse", bound=256)
    codes = unpack_codes(packed).reshape(128, 4, 16)
    blocks = x.reshape(128, 4, 16).astype(np.float64)
    a = np.abs(blocks).max(axis=2)
    s6 = oracle.E4M3_VALUES[oracle.e4m3_encode(np.fmin((a / 6).astype(F32), 448))]
    s4 = oracle.E4M3_VALUES[oracle.e4m3_encode(np.fmin(((a / 6).astype(F32) * F32(1.5)), 448))]
    s = oracle.E4M3_VALUES[scales]
    assert np.all((s == s6) | (s == s4))
    deq = code_values(codes).astype(np.float64) * s[..., None]
    chosen = ((blocks - deq) ** 2).sum(axis=2)
    for sc in (s6, s4):
        other = oracle.e2m1_rtn_index(np.abs(blocks).astype(F32) * (F32(1) / sc.astype(F32))[..., None])
        alt = np.sign(blocks) * oracle.E2M1_GRID[other] * sc[..., None]
        err = ((blocks - alt) ** 2).sum(axis=2)
        clear = np.abs(err - chosen) > 1e-4 * np.maximum(err, chosen)
        assert np.all(chosen[clear] <= err[clear])


# --------------------------------------------------------------- 2D blocks

@pytest.mark.parametrize("global_scale", [False, True])
def test_2d_scale_is_transposition_invariant(global_scale):
    # Stable FP4 Training via Transposition-Invariant Block Quantization:
    # one scale per 16x16 tile, identical for X and X^T.
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 96)) * np.exp(rng.uniform(-3, 3, (64, 96)))).astype(F32)
    xt = np.ascontiguousarray(x.T)
    A = oracle.amax(x) if global_scale else None
    r, c, s = oracle.quantize_2d(x, global_amax=A)
    rt, ct, st = oracle.quantize_2d(xt, global_amax=A)
    assert np.array_equal(st, s.T)
    assert np.array_equal(c, rt) and np.array_equal(ct, r)  # RTN: col(X) == row(X^T)
    r2, c2, _ = oracle.quantize_2d(x, stochastic=True, seed=3, step=5, global_amax=A)
    assert np.array_equal(c2, oracle.nvfp4.pack_codes(unpack_codes(r2).T))


def test_2d_tile_scale_bounds_every_element():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((32, 32)).astype(F32)
    x[3, 17] = 40.0
    r, _, s = oracle.quantize_2d(x)
    assert s[0, 1] == oracle.e4m3_encode(F32(40.0) / F32(6.0))
    assert unpack_codes(r)[3, 17] == 0x7


# -------------------------------------------------- zero and tiny blocks

def test_zero_and_sub_range_blocks_dequantize_to_zero():
    # fp4-train, Requirements and limits: a block whose absmax is below the
    # e4m3 scale range quantizes to zero.  a <= 6 * 2**-10 -> sigma <= 2**-10,
    # half the smallest e4m3 step, which rounds (ties to even) to scale byte
    # 0 -> x_hat = +-0, and the residual keeps x' exactly.  Just above, the
    # scale is the smallest subnormal 2**-9 (byte 0x01).
    x = np.zeros((1, 48), F32)
    x[0, 16:32] = np.linspace(-6 * 2.0 ** -10, 6 * 2.0 ** -10, 16)
    x[0, 32:48] = 6 * 2.0 ** -10 * 1.01
    r = np.zeros_like(x)
    out, packed, scales = oracle.qdq(x, residual=r, out="f32")
    assert scales[0].tolist()[:2] == [0, 0] and scales[0, 2] == 1
    assert np.all(unpack_codes(packed)[0, :16] == 0)
    assert np.all(out[0, :32] == 0)
    assert np.array_equal(r[0, :32], x[0, :32])


# ----------------------------------------------------------- special values

def test_nan_inputs():
    # CuTe DSL kernel Design / Bitwise validation: NaN-dropping block amax,
    # NaN encodes to +6 (code 0x7), an all-NaN block has amax 0.
    x = np.zeros((1, 32), F32)
    x[0, :16] = np.linspace(-3, 3, 16)
    ref_p, ref_s = oracle.quantize(x)
    x[0, 5] = np.nan
    x[0, 16:] = np.nan
    p, s = oracle.quantize(x)
    codes, ref_codes = unpack_codes(p)[0], unpack_codes(ref_p)[0]
    assert s[0, 0] == ref_s[0, 0] and s[0, 1] == 0
    assert codes[5] == 0x7 and np.array_equal(np.delete(codes[:16], 5), np.delete(ref_codes[:16], 5))
    assert np.all(codes[16:] == 0x7)
    p6, s6 = oracle.quantize_4over6(x, oracle.amax(x), bound=256)
    assert unpack_codes(p6)[0, 5] == 0x7


def test_inf_inputs():
    x = np.zeros((1, 16), F32)
    x[0, :3] = [np.inf, -np.inf, 1.0]
    p, s = oracle.quantize(x)
    assert s[0, 0] == 0x7E  # sigma = inf is capped to 448
    assert unpack_codes(p)[0, :3].tolist() == [0x7, 0xF, 0x0]
    # amax == inf with a global scale: S_enc = 0, so finite blocks get scale
    # 0 and rho = min(1/(0*inf), FLT_MAX) = FLT_MAX.
    y = np.ones((1, 32), F32)
    y[0, 0] = np.inf
    p, s = oracle.quantize_4over6(y, oracle.amax(y), bound=256)
    assert s[0, 1] == 0 and np.all(unpack_codes(p)[0, 16:] == 0x7)


def test_empty_inputs():
    x = np.zeros((0, 32), F32)
    p, s = oracle.quantize(x)
    assert p.shape == (0, 16) and s.shape == (0, 2)
    assert oracle.amax(x) == 0


@pytest.mark.parametrize("nan_bits", [0x7F800001, 0xFF812345, 0x7FC00000, 0xFFC00000, 0x7FBFFFFF])
@pytest.mark.parametrize("pos", [0, 5, 15])
def test_nan_dropping_amax_drops_every_nan(nan_bits, pos):
    """Block, row and tensor amaxes drop NaNs, signalling ones included,
    wherever they sit: the amax is the max magnitude of the other elements
    (and 0 for an all-NaN group).  Brute force over the finite elements."""
    rng = np.random.default_rng(nan_bits % 1000 + pos)
    x = (rng.standard_normal((3, 32)) * 100).astype(F32)
    x[:, 7] = F32(-812.5)                      # the largest magnitude sits before the NaN
    x.view(np.uint32)[:, 16 + pos] = nan_bits
    x.view(np.uint32)[1, 8 + pos // 2] = nan_bits
    x.view(np.uint32)[2, :16] = nan_bits       # an all-NaN block
    fin = np.where(np.isnan(x), F32(0), np.abs(x))
    assert np.array_equal(oracle.amax(x, mode="row"), fin.max(axis=1))
    assert oracle.amax(x) == fin.max()
    _, s = oracle.quantize(x)
    want = oracle.e4m3_encode(np.fmin(fin.reshape(3, 2, 16).max(axis=2) / F32(6), F32(448)))
    assert np.array_equal(s, want)
    assert s[2, 0] == 0
