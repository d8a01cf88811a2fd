"""The C ABI without a GPU: the library loads, exports every entry point that
include/nvfp4.h declares, and rejects bad arguments on the host with the
documented status before anything is launched (fake, never-dereferenced
device addresses are passed; no compute call is made)."""
import ctypes
import os
import re

import pytest

from fp4_block_quantization_nvfp4_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "nvfp4.h")
A = 1 << 20  # a fake, 256-byte-aligned device address (never dereferenced)


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert {"nvfp4_quantize", "nvfp4_dequantize", "nvfp4_qdq", "nvfp4_quantize_4over6",
            "nvfp4_quantize_2d", "nvfp4_amax"} <= set(names)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES)


def test_status_strings():
    for s in range(8):
        assert L.status_str(s)
    assert L.status_str(99) == "unknown status"


def q(*, x=A, dt=L.BF16, M=32, K=64, res=None, ga=None, rnd=L.RTN, packed=A, scales=A):
    return L.lib().nvfp4_quantize(x, dt, M, K, res, ga, rnd, 0, 0, packed, scales, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=24), L.E_SHAPE), (dict(M=-1), L.E_SHAPE), (dict(K=-16), L.E_SHAPE),
    (dict(dt=7), L.E_DTYPE), (dict(rnd=5), L.E_ARG), (dict(x=None), L.E_NULL),
    (dict(packed=None), L.E_NULL), (dict(scales=None), L.E_NULL),
    (dict(x=A + 8), L.E_ALIGN), (dict(res=A + 4), L.E_ALIGN), (dict(packed=A + 4), L.E_ALIGN),
    (dict(ga=A + 2), L.E_ALIGN), (dict(M=1 << 22, K=1 << 12), L.E_RANGE),
])
def test_quantize_rejects(kw, status):
    assert q(**kw) == status


def test_empty_is_ok_without_pointers():
    assert q(x=None, packed=None, scales=None, M=0) == L.OK
    assert q(x=None, packed=None, scales=None, K=0) == L.OK


def test_other_entry_points_reject():
    lib = L.lib()
    # dequantize: tile16 needs M % 16; bad bound with a global scale; NULL out
    assert lib.nvfp4_dequantize(A, A, 8, 32, 1, None, 0, 448.0, A, L.BF16, None) == L.E_SHAPE
    assert lib.nvfp4_dequantize(A, A, 16, 32, 0, A, 1, 300.0, A, L.BF16, None) == L.E_ARG
    assert lib.nvfp4_dequantize(A, A, 16, 32, 0, None, 0, 448.0, None, L.BF16, None) == L.E_NULL
    assert lib.nvfp4_dequantize(A, A, 16, 32, 1, A, 2, 448.0, A, L.BF16, None) == L.E_ARG
    # qdq: bad out dtype
    assert lib.nvfp4_qdq(A, L.BF16, 4, 32, None, None, 0, 0, 0, A, 9, None, None, None) == L.E_DTYPE
    assert lib.nvfp4_qdq(A, L.BF16, 4, 32, None, None, 0, 0, 0, A, L.BF16, A, None, None) == L.E_NULL
    # four-over-six: bound, err, mode, per-tensor must be given
    assert lib.nvfp4_quantize_4over6(A, L.BF16, 4, 32, A, 1, 1, 0, 300.0, A, A, None) == L.E_ARG
    assert lib.nvfp4_quantize_4over6(A, L.BF16, 4, 32, A, 1, 1, 3, 256.0, A, A, None) == L.E_ARG
    assert lib.nvfp4_quantize_4over6(A, L.BF16, 4, 32, A, 0, 1, 0, 256.0, A, A, None) == L.E_ARG
    assert lib.nvfp4_quantize_4over6(A, L.BF16, 4, 32, A, 1, 0, 0, 256.0, A, A, None) == L.E_ARG
    assert lib.nvfp4_quantize_4over6(A, L.BF16, 4, 32, None, 2, 0, 0, 256.0, A, A, None) == L.E_NULL
    # 2D: M % 16
    assert lib.nvfp4_quantize_2d(A, L.BF16, 24, 32, None, 0, 0, 0, 0, A, A, A, None) == L.E_SHAPE
    assert lib.nvfp4_quantize_2d(A, L.BF16, 32, 32, None, 0, 0, 0, 0, None, A, A, None) == L.E_NULL
    assert lib.nvfp4_quantize_2d(A, L.BF16, 32, 32, None, 0, 0, 0, 2, A, A, A, None) == L.E_ARG
    # rowcol: M % 16, standard path needs bound 448, four-over-six 256/448, amax required
    rc = lib.nvfp4_quantize_rowcol
    assert rc(A, L.BF16, 24, 32, A, 0, 0, 448.0, A, A, A, A, None) == L.E_SHAPE
    assert rc(A, L.BF16, 32, 32, A, 0, 0, 256.0, A, A, A, A, None) == L.E_ARG
    assert rc(A, L.BF16, 32, 32, A, 1, 0, 300.0, A, A, A, A, None) == L.E_ARG
    assert rc(A, L.BF16, 32, 32, A, 2, 0, 448.0, A, A, A, A, None) == L.E_ARG
    assert rc(A, L.BF16, 32, 32, A, 1, 4, 256.0, A, A, A, A, None) == L.E_ARG
    assert rc(A, L.BF16, 32, 32, None, 1, 0, 256.0, A, A, A, A, None) == L.E_NULL
    assert rc(A, L.BF16, 32, 32, A, 1, 0, 256.0, A, A, None, A, None) == L.E_NULL
    assert rc(A, L.BF16, 32, 32, A, 1, 0, 256.0, A, A, A + 4, A, None) == L.E_ALIGN
    assert rc(None, L.BF16, 0, 32, None, 1, 0, 256.0, None, None, None, None, None) == L.OK
    # four-over-six 16x16: M % 16, bound, err, amax required, column output optional
    f2 = lib.nvfp4_quantize_4over6_2d
    assert f2(A, L.BF16, 8, 32, A, 0, 256.0, A, A, A, None) == L.E_SHAPE
    assert f2(A, L.BF16, 16, 32, A, 0, 100.0, A, A, A, None) == L.E_ARG
    assert f2(A, L.BF16, 16, 32, A, 2, 256.0, A, A, A, None) == L.E_ARG
    assert f2(A, L.BF16, 16, 32, None, 0, 256.0, A, A, A, None) == L.E_NULL
    assert f2(A, L.BF16, 16, 32, A, 0, 256.0, A, A, None, None) == L.E_NULL
    assert f2(A, 3, 16, 32, A, 0, 256.0, A, A, A, None) == L.E_DTYPE
    # amax: workspace too small / missing, bad mode
    need = lib.nvfp4_amax_workspace_bytes(1024, 1024)
    assert need >= 4
    assert lib.nvfp4_amax(A, L.BF16, 1024, 1024, None, 1, A, A, need - 1, None) == L.E_ARG
    assert lib.nvfp4_amax(A, L.BF16, 1024, 1024, None, 1, A, None, need, None) == L.E_NULL
    assert lib.nvfp4_amax(A, L.BF16, 1024, 1024, None, 0, A, A, need, None) == L.E_ARG


def test_selftest_scan_rejects():
    s = L.lib().nvfp4_selftest_scan
    assert s(5, 0, 0, 16, 4, A, None) == L.E_ARG            # unknown kind
    assert s(-1, 0, 0, 16, 4, A, None) == L.E_ARG
    assert s(0, 0, 0, 16, 25, A, None) == L.E_ARG           # chunk too large
    assert s(0, 0, 0, 1 << 32, 8, A, None) == L.E_ARG       # 2^24 chunks > 2^22
    assert s(0, 0, 1, 1 << 32, 16, A, None) == L.E_RANGE    # past the pattern space
    assert s(0, 0, (1 << 32) + 1, 0, 16, A, None) == L.E_RANGE
    assert s(3, 0, 0, 257, 0, A, None) == L.E_RANGE         # decodes take bytes only
    assert s(0, 0, 0, 16, 4, None, None) == L.E_NULL
    assert s(0, 0, 0, 16, 4, A + 8, None) == L.E_ALIGN
    assert s(0, 0, 0, 0, 4, None, None) == L.OK             # empty run


def _plan(entry, M, K, bf16=1, variant=0):
    out = (ctypes.c_int64 * 4)()
    st = L.lib().nvfp4_selftest_launch_plan(entry, M, K, bf16, variant, out)
    return st, list(out)


@pytest.mark.parametrize("entry,variant", [(0, 0), (1, 0), (1, 1), (2, 0), (3, 0), (4, 0), (4, 1), (5, 0),
                                           (5, 1), (6, 0), (6, 1)])
@pytest.mark.parametrize("bf16", [0, 1])
def test_launch_geometry_within_dispatch_limits(entry, variant, bf16):
    """Every accepted shape, down to 16-element rows with the largest M the
    2^33-element limit allows (the case where one workgroup per row would
    exceed 2^32 work-items), keeps each launch under 2^32 work-items and
    2^31 workgroups and covers all rows."""
    for K in (16, 32, 128, 320, 7168, 16384, 16400, 65536, 1 << 20, 1 << 33):
        for M in (16, 8192, 1 << 25, (1 << 25) + 16, 1 << 26, (1 << 33) // K // 16 * 16):
            if M * K > 1 << 33 or M < 1:
                continue
            st, (kern, launches, grid, block) = _plan(entry, M, K, bf16, variant)
            assert st == L.OK, (entry, M, K)
            assert 1 <= grid < 1 << 31 and 64 <= block <= 1024 and grid * block < 1 << 32, (entry, M, K, grid, block)
            if kern == 2:  # the bf16 row kernel: one workgroup per row, in chunks
                assert bf16 and K <= 16384 and launches * grid >= M and grid * (launches - 1) < M
            else:
                assert launches == 1
    assert _plan(2, 1 << 26, 16)[1][:2] == [2, 4]             # 2^26 rows: four row-kernel launches
    assert _plan(2, 8192, 7168)[1] == [2, 1, 8192, 128]      # the metric shape
    assert _plan(2, 8192, 7168, bf16=0)[1][0] == 3           # fp32 takes the generic kernel
    assert _plan(3, 24, 32)[0] == L.E_SHAPE and _plan(7, 16, 16)[0] == L.E_ARG
    assert _plan(0, 1 << 22, 1 << 12)[0] == L.E_RANGE


def test_tile_kernel_strips_per_workgroup():
    """The 16x16 four-over-six kernel walks 16 strips per workgroup with the
    columnwise output; rowwise only it takes the largest of 16, 8 and 4
    strips that still gives 1024 workgroups (else 4), so small tensors fill
    the chip."""
    def grid(M, K, col):
        st, (kern, launches, g, block) = _plan(5, M, K, 1, col)
        assert st == L.OK and kern == 6 and block == 512
        return g
    xcd = lambda n: 8 * ((n + 7) // 8)
    assert grid(7168, 18432, 1) == xcd(36 * 28)       # columnwise: 16 strips
    assert grid(8192, 7168, 1) == xcd(14 * 32)
    assert grid(8192, 7168, 0) == xcd(14 * 128)       # rowwise: 4 strips
    assert grid(8192, 2048, 0) == xcd(4 * 128)
    assert grid(32768, 2048, 0) == xcd(4 * 256)       # 8 strips reach 1024
    assert grid(131072, 7168, 0) == xcd(14 * 512)     # 16 strips


def test_amax_noalloc_rejects():
    f = L.lib().nvfp4_amax_noalloc
    assert f(A, L.BF16, 1024, 1024, None, 0, A, None) == L.E_ARG       # mode NONE
    assert f(A, L.BF16, 1024, 1000, None, 1, A, None) == L.E_SHAPE
    assert f(A, 5, 1024, 1024, None, 1, A, None) == L.E_DTYPE
    assert f(A, L.BF16, 1024, 1024, None, 1, None, None) == L.E_NULL
    assert f(None, L.BF16, 1024, 1024, None, 1, A, None) == L.E_NULL
    assert f(A + 4, L.BF16, 1024, 1024, None, 1, A, None) == L.E_ALIGN
    assert f(A, L.BF16, 1 << 22, 1 << 12, None, 1, A, None) == L.E_RANGE  # M*K > 2^33
