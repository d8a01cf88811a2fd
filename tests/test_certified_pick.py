"""The four-over-six kernels decide most blocks from approximate error sums
in the scaled domain plus a rounding margin, instead of the pages' exact
rule (four-over-six pull request, CuTe DSL kernel Design: true divisions by
6 * bound, element-order sums, the width-16 tree for tiles, strict
err4 < err6).  This CPU test runs a replica of that shortcut
(tests/c/fos_check.c, fp32 with the kernels' fma placement) on blocks and
tiles driven by bisection to the exact decision boundary, where a margin
that is too small would flip a pick:

* every decided pick equals the exact rule's pick;
* the exact sums the kernels use for undecided blocks equal the exact
  rule's sums bit for bit, and the identical-dequant test only fires on
  exact ties;
* the rounding uses at most 1/2.6 of the margin (the derivation's safety
  factor), reported as worst_margin_use.

The replica's exact rule is in turn compared with the oracle on the
bracketing blocks it writes, so the boundary blocks are the oracle's.
"""
import numpy as np
import pytest

import oracle
from oracle.formats import FLT_MAX
from tests import fos_records


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    return fos_records.build(tmp_path_factory.mktemp("fos"))


@pytest.mark.parametrize("mode,n,seed", [("1x16", 100000, 1), ("tile", 8000, 2)])
def test_certified_pick_never_contradicts_the_exact_rule(exe, mode, n, seed):
    rc, text = fos_records.run(exe, mode, n, seed)
    assert rc == 0, text
    s = fos_records.summary(text)
    assert s["failures"] == 0
    assert s["decided"] > 0 and s["undecided"] > 0 and s["same_dequant"] > 0
    assert s["worst_margin_use"] < 1 / 2.6, text


def _oracle_pick4_rows(x, A, bound, mse):
    """Map-to-4 flags of single-block rows with per-row amax A, from the
    oracle's scale bytes (rows where both candidates share a scale byte are
    reported as None: the pick is invisible there)."""
    p, s = oracle.quantize_4over6(x, A, err_mode="mse" if mse else "mae", bound=bound)
    D = np.float32(6 * bound)
    a = np.abs(x).max(axis=1)
    S_enc = np.fmin(D / A, FLT_MAX)
    sig6 = (a / np.float32(6.0)) * S_enc
    k6 = oracle.e4m3_encode(np.fmin(sig6, np.float32(448)))
    k4 = oracle.e4m3_encode(np.fmin(sig6 * np.float32(1.5), np.float32(448)))
    return s[:, 0] == k4, k4 != k6


def test_replica_exact_rule_is_the_oracles_1x16(exe, tmp_path):
    out = tmp_path / "blocks.bin"
    rc, text = fos_records.run(exe, "1x16", 3000, 11, out)
    assert rc == 0, text
    x, A, bound, mse, bf16, pick4 = fos_records.read(out, 16)
    assert len(x) > 500
    for b in (256.0, 448.0):
        for m in (False, True):
            sel = (bound == b) & (mse == m)
            got, visible = _oracle_pick4_rows(x[sel], A[sel], b, m)
            assert np.array_equal(got[visible], pick4[sel][visible])
            assert visible.mean() > 0.5


def test_replica_exact_rule_is_the_oracles_tiles(exe, tmp_path):
    out = tmp_path / "tiles.bin"
    rc, text = fos_records.run(exe, "tile", 3000, 12, out, A=30000.0)
    assert rc == 0, text
    x, A, bound, mse, bf16, pick4 = fos_records.read(out, 256)
    assert len(x) > 100 and np.all(A == np.float32(30000.0))
    n_vis = 0
    for b in (256.0, 448.0):
        for m in (False, True):
            sel = np.flatnonzero((bound == b) & (mse == m))
            if len(sel) == 0:
                continue
            t = x[sel].reshape(-1, 16, 16)
            wide = np.ascontiguousarray(t.transpose(1, 0, 2).reshape(16, -1))  # tiles side by side
            p, s = oracle.quantize_4over6(wide, np.float32(30000.0), err_mode="mse" if m else "mae", bound=b,
                                          block="16x16")
            a = np.abs(t).max(axis=(1, 2))
            sig6 = (a / np.float32(6.0)) * np.fmin(np.float32(6 * b) / np.float32(30000.0), FLT_MAX)
            k6 = oracle.e4m3_encode(np.fmin(sig6, np.float32(448)))
            k4 = oracle.e4m3_encode(np.fmin(sig6 * np.float32(1.5), np.float32(448)))
            vis = k4 != k6
            assert np.array_equal((s[0] == k4)[vis], pick4[sel][vis])
            n_vis += int(vis.sum())
    assert n_vis > 0.5 * len(x)
