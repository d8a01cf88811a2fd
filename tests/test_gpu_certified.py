"""GPU parity on adversarial four-over-six inputs: blocks and tiles moved by
bisection to the exact decision boundary (tests/c/fos_check.c; each record
is one of the two adjacent values where the exact pick flips), so that a
certified margin that is too small, or a wrong exact fallback, shows up as a
mismatch.  Every output is compared bit for bit with the oracle (four-over-six
pull request, CuTe DSL kernel Design: true divisions by 6 * bound,
element-order sums, the width-16 tree, strict err4 < err6).

* 1x16 blocks, one block per row with its own row amax given (the bf16 row
  kernel and the generic fp32 kernel), and with the row amax computed in
  the pass where the record's amax is the block's own;
* 1x16 blocks under one per-tensor amax: the per-tensor path and the fused
  row + column pass (rowwise blocks are the records);
* 16x16 tiles under one per-tensor amax (rowwise, columnwise and scales).
"""
import numpy as np
import pytest
import torch

import oracle
import fp4_block_quantization_nvfp4_amd as nv
from tests import fos_records
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

FIXED_A = np.float32(30000.0)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(scope="module")
def records(tmp_path_factory):
    d = tmp_path_factory.mktemp("fos")
    exe = fos_records.build(d)
    out = {}
    for name, mode, n, seed, A in (("rows", "1x16", 20000, 21, None), ("tensor", "1x16", 20000, 22, FIXED_A),
                                   ("tiles", "tile", 24000, 23, FIXED_A)):
        path = d / f"{name}.bin"
        rc, text = fos_records.run(exe, mode, n, seed, path, A)
        assert rc == 0, text
        out[name] = fos_records.read(path, 256 if mode == "tile" else 16)
    return out


def _groups(rec):
    x, A, bound, mse, bf16, _ = rec
    for b in (256.0, 448.0):
        for m in (False, True):
            for h in (False, True):
                sel = (bound == b) & (mse == m) & (bf16 == h)
                if sel.any():
                    xs = np.ascontiguousarray(x[sel])
                    xin = (xs.view(np.uint32) >> 16).astype(np.uint16) if h else xs
                    yield xin, A[sel], b, ("mse" if m else "mae"), f"bound={b} {'mse' if m else 'mae'} {'bf16' if h else 'f32'}"


def test_boundary_blocks_row_amax(records):
    n = 0
    for xin, A, b, err, what in _groups(records["rows"]):
        wp, ws = oracle.quantize_4over6(xin, A, err_mode=err, bound=b)
        p, s, _ = nv.quantize_4over6(to_dev(xin), torch.from_numpy(A).cuda(), err_mode=err,
                                     e4m3_scale_bound=int(b), row_scaled=True)
        assert_bitwise(to_np(s), ws, f"scales {what}")
        assert_bitwise(to_np(p), wp, f"codes {what}")
        # records whose amax is the block's own: the row amax computed in the pass
        own = np.abs(oracle.bf16_bits_to_f32(xin) if xin.dtype == np.uint16 else xin).max(axis=1) == A
        if own.sum() >= 1:
            xo = np.ascontiguousarray(xin[own])
            p, s, Ad = nv.quantize_4over6(to_dev(xo), None, err_mode=err, e4m3_scale_bound=int(b), row_scaled=True)
            assert_bitwise(to_np(Ad), A[own], f"row amax {what}")
            assert_bitwise(to_np(s), ws[own], f"scales (amax computed) {what}")
            assert_bitwise(to_np(p), wp[own], f"codes (amax computed) {what}")
        n += len(xin)
    assert n > 5000


def test_boundary_blocks_per_tensor_and_rowcol(records):
    n = 0
    for xin, A, b, err, what in _groups(records["tensor"]):
        assert np.all(A == FIXED_A)
        wp, ws = oracle.quantize_4over6(xin, FIXED_A, err_mode=err, bound=b)
        Ad = torch.tensor([FIXED_A], dtype=torch.float32, device="cuda")
        p, s, _ = nv.quantize_4over6(to_dev(xin), Ad, err_mode=err, e4m3_scale_bound=int(b), row_scaled=False)
        assert_bitwise(to_np(s), ws, f"scales {what}")
        assert_bitwise(to_np(p), wp, f"codes {what}")
        R = len(xin) // 16 * 16
        if R:
            xr = np.ascontiguousarray(xin[:R])
            got = [to_np(t) for t in nv.quantize_rowcol(to_dev(xr), Ad, four_over_six=True, err_mode=err,
                                                         e4m3_scale_bound=int(b))]
            want = oracle.quantize_rowcol(xr, FIXED_A, four_over_six=True, err_mode=err, bound=b)
            for g, w, nm in zip(got, want, ("row codes", "row scales", "col codes", "col scales")):
                assert_bitwise(g, w, f"rowcol {nm} {what}")
        n += len(xin)
    assert n > 5000


def test_boundary_tiles(records):
    n = 0
    for xin, A, b, err, what in _groups(records["tiles"]):
        t = xin.reshape(-1, 16, 16)
        wide = np.ascontiguousarray(t.transpose(1, 0, 2).reshape(16, -1))
        wr, wc, wt = oracle.quantize_4over6_2d(wide, FIXED_A, err_mode=err, bound=b)
        Ad = torch.tensor([FIXED_A], dtype=torch.float32, device="cuda")
        r, c, ts = nv.quantize_4over6_2d(to_dev(wide), Ad, err_mode=err, e4m3_scale_bound=int(b))
        assert_bitwise(to_np(ts), wt, f"tile scales {what}")
        assert_bitwise(to_np(r), wr, f"rowwise {what}")
        assert_bitwise(to_np(c), wc, f"columnwise {what}")
        n += len(t)
    assert n > 500
