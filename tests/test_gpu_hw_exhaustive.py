"""Exhaustive checks of the gfx950 conversions behind the element codes and
scale bytes, against the oracle, over every input bit pattern.

nvfp4_selftest_scan runs the kernels' own device helpers over a run of
patterns and reports, per chunk of 2^16 consecutive patterns, the output at
both ends, how many times the output changes inside the chunk, and where it
first changes.  The oracle's encoders are monotone in the pattern within each
sign half (round-to-nearest-even onto a sorted grid; stochastic rounding with
a fixed draw rounds up on a suffix of every grid interval).  So if the GPU's
output equals the oracle's at every chunk end, changes at most once inside a
chunk, and the oracle takes the GPU's values on both sides of that change,
then the two agree on every pattern of the run.  Covered:

* fp32 -> e2m1 round-to-nearest-even, saturating (the pages: satfinite RNE
  casts, four-over-six pull request, CuTe DSL kernel Design), for every
  non-NaN fp32 value of either sign, in each byte position and element slot
  the kernels use; the other bytes of the word must come back unchanged.
  NaN inputs never reach it (blocks with a NaN take the software encoder);
  the hardware's NaN codes (0x7 for +NaN, 0xF for -NaN) are asserted as
  documented behaviour.
* fp32 -> e4m3 of min(sigma, 448), both slots, for every pattern with the
  sign bit clear (all non-negative values, +inf and NaN).
* stochastic fp32 -> e2m1 (fp4-train card, Method: round up with probability
  equal to the fractional distance; the oracle's reading compares the draw
  with that distance truncated to 22 bits) for every non-NaN fp32 value of
  either sign under 44 draws that include 0, 1, 2^k, 2^k - 1 and 0xFFFF, in
  both slots (byte 0), and four draws in every other byte position.
* the e2m1 -> fp32 decode of all 256 bytes (both halves, every byte
  position) and the e4m3 -> fp32 decode of the 127 scale codes.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.nvfp4 import _encode
from fp4_block_quantization_nvfp4_amd import _lib as L
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

F32 = np.float32
CH = 16                      # chunk_log2
HALF = 0x7F800001            # non-NaN patterns of one sign: 0 .. +inf
OLD = 0xA5A5A5A5


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def scan(kind, param, first, count, chunk_log2=CH):
    n = (count + (1 << chunk_log2) - 1) >> chunk_log2
    rec = torch.empty(n * 4, dtype=torch.int32, device="cuda")
    L.check(L.lib().nvfp4_selftest_scan(kind, param, first, count, chunk_log2, rec.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream), "nvfp4_selftest_scan")
    return rec.cpu().numpy().view(np.uint32).reshape(n, 4)


def verify(rec, first, count, expected, what, chunk_log2=CH):
    n = len(rec)
    starts = first + (np.arange(n, dtype=np.int64) << chunk_log2)
    ends = np.minimum(starts + (1 << chunk_log2), first + count) - 1
    e0 = expected(starts.astype(np.uint32))
    e1 = expected(ends.astype(np.uint32))
    assert np.array_equal(rec[:, 0], e0), f"{what}: chunk starts"
    assert np.array_equal(rec[:, 1], e1), f"{what}: chunk ends"
    assert np.all(rec[:, 2] <= 1), f"{what}: more than one change in a chunk"
    one = rec[:, 2] == 1
    pos = rec[one, 3].astype(np.int64)
    assert np.all((pos > starts[one]) & (pos <= ends[one]))
    assert np.array_equal(expected((pos - 1).astype(np.uint32)), rec[one, 0]), f"{what}: before a change"
    assert np.array_equal(expected(pos.astype(np.uint32)), rec[one, 1]), f"{what}: after a change"
    assert np.all(rec[~one, 0] == rec[~one, 1])
    # changes inside chunks plus changes exactly at a chunk's first pattern
    return int(one.sum()) + int(np.count_nonzero(rec[1:, 0] != rec[:-1, 1]))


def _codes(p, u16=None):
    x = p.view(F32)
    code, _ = _encode(x, F32(1.0), None if u16 is None else np.full(x.shape, u16))
    return code.astype(np.uint32)


def _word(code, sel, slot_b):
    byte = (code << 4) if slot_b else code
    return ((OLD & ~(0xFF << (8 * sel))) | (byte << (8 * sel))).astype(np.uint32)


@pytest.mark.parametrize("sel", range(4))
@pytest.mark.parametrize("slot_b", [False, True], ids=["a", "b"])
def test_e2m1_round_to_nearest_every_fp32(sel, slot_b):
    changes = 0
    for first in (0, 0x80000000):
        rec = scan(0, sel | (slot_b << 2), first, HALF)
        changes += verify(rec, first, HALF, lambda p: _word(_codes(p), sel, slot_b), f"rtn sel={sel}")
    assert changes == 14  # seven thresholds per sign
    # NaN inputs (kept off this path by the kernels): +NaN -> 0x7, -NaN -> 0xF
    for first, code in ((0x7F800001, 0x7), (0xFF800001, 0xF)):
        rec = scan(0, sel | (slot_b << 2), first, 0x7FFFFF)
        assert np.all(rec[:, 2] == 0) and np.all(rec[:, 0] == _word(np.uint32(code), sel, slot_b))


@pytest.mark.parametrize("slot", [0, 1])
def test_e4m3_scale_every_nonnegative_fp32(slot):
    want = lambda p: oracle.e4m3_encode(np.fmin(p.view(F32), F32(448.0))).astype(np.uint32)
    rec = scan(1, slot, 0, 0x80000000)
    assert verify(rec, 0, 0x80000000, want, f"e4m3 slot {slot}") == 126


DRAWS = sorted({0, 1, 2, 3, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF, 12345, 40000, 0xBEEF,
                *[1 << k for k in range(1, 16)], *[(1 << k) - 1 for k in range(2, 16)],
                *np.random.default_rng(9).integers(0, 1 << 16, 7).tolist()})


@pytest.mark.parametrize("slot_b", [False, True], ids=["a", "b"])
def test_stochastic_e2m1_every_fp32_fixed_draws(slot_b):
    assert len(DRAWS) >= 40
    for u in DRAWS:
        sels = range(4) if u in (0, 0x8000, 0xFFFF, 12345) else (0,)
        for sel in sels:
            for first in (0, 0x80000000):
                rec = scan(2, u | (sel << 16) | (slot_b << 18), first, HALF)
                want = lambda p: ((_codes(p, u) << 4) if slot_b else _codes(p, u)).astype(np.uint32)
                verify(rec, first, HALF, want, f"sr u={u} sel={sel}")


def test_decodes_exhaustive():
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], F32)
    b = np.arange(256, dtype=np.uint32)
    for sel in range(4):
        for half in (0, 1):
            rec = scan(3, sel | (half << 2), 0, 256, chunk_log2=0)
            nib = (b >> 4) if half else (b & 0xF)
            want = np.where(nib & 8, -grid[nib & 7], grid[nib & 7]).astype(F32).view(np.uint32)
            assert np.array_equal(rec[:, 0], want), (sel, half)
    for sel in (0, 1):
        rec = scan(4, sel, 0, 127, chunk_log2=0)
        assert np.array_equal(rec[:, 0], oracle.e4m3_decode(np.arange(127)).view(np.uint32)), sel
