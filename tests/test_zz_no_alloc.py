"""The allocation-free amax entry point (nvfp4_amax_noalloc), through the C
ABI, against the workspace entry point (nvfp4_amax) and the oracle, bit for
bit: two calls in a row on one GPU, the second with a smaller input (the
shared scratch array keeps the first call's partials), per tensor and per
row, bf16 and fp32, with and without a residual."""
import numpy as np
import pytest
import torch

import oracle
from fp4_block_quantization_nvfp4_amd import _lib as L
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, wide_input

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _both(x, r, mode):
    lib, st = L.lib(), torch.cuda.current_stream().cuda_stream
    M, K = x.shape
    dt = L.BF16 if x.dtype == torch.bfloat16 else L.F32
    n = 1 if mode == L.SCALE_TENSOR else M
    ws_bytes = lib.nvfp4_amax_workspace_bytes(M, K)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    ref = torch.full((n,), -1.0, dtype=torch.float32, device="cuda")
    got = torch.full((n,), -2.0, dtype=torch.float32, device="cuda")
    rp = r.data_ptr() if r is not None else None
    L.check(lib.nvfp4_amax(x.data_ptr(), dt, M, K, rp, mode, ref.data_ptr(), ws.data_ptr(), ws_bytes, st),
            "nvfp4_amax")
    L.check(lib.nvfp4_amax_noalloc(x.data_ptr(), dt, M, K, rp, mode, got.data_ptr(), st), "nvfp4_amax_noalloc")
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("mode", [L.SCALE_TENSOR, L.SCALE_ROW], ids=["tensor", "row"])
@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
@pytest.mark.parametrize("with_res", [False, True], ids=["plain", "residual"])
def test_noalloc_amax_matches_workspace_entry_point(mode, bf16, with_res):
    for i, (M, K) in enumerate(((4096, 7168), (48, 1040))):  # the second call is smaller
        x = wide_input(100 + i, M, K, bf16=bf16)
        xd = to_dev(x)
        r = (np.random.default_rng(200 + i).standard_normal((M, K)) * 1e-2).astype(np.float32) if with_res else None
        rd = torch.from_numpy(r).cuda() if with_res else None
        ref, got = _both(xd, rd, mode)
        assert_bitwise(got, ref, f"call {i}: noalloc vs workspace amax")
        want = oracle.amax(x, residual=r, mode="tensor" if mode == L.SCALE_TENSOR else "row")
        assert_bitwise(got, np.atleast_1d(np.asarray(want, np.float32)), f"call {i}: noalloc vs oracle")
