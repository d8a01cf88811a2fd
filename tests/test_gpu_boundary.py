"""The bf16 four-over-six row kernel (one workgroup per row) is launched in
chunks of at most 2^24 rows, so that no launch exceeds the dispatch limit of
2^32 work-items (fp4-train card, Requirements and limits: any M with K a
multiple of 16).  This runs a tensor of 2^24 + 48 rows of 16 elements (two
launches) and compares the rows on both sides of the chunk boundary, the
first and last rows and a random sample with the oracle, and the row amax of
every row."""
import numpy as np
import pytest
import torch

import oracle
import fp4_block_quantization_nvfp4_amd as nv
from tests.gpu_util import assert_bitwise, need_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("amax_given", [False, True], ids=["computed", "given"])
def test_row_kernel_two_launches(amax_given):
    M, K = (1 << 24) + 48, 16
    rng = np.random.default_rng(5)
    xd = torch.randn((M, K), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda",
                     dtype=torch.float32)
    xd = (xd * torch.exp2(torch.linspace(-20, 20, M, device="cuda"))[:, None]).to(torch.bfloat16)
    x = xd.view(torch.int16).cpu().numpy().view(np.uint16)
    wA = oracle.amax(x, mode="row")
    A = torch.from_numpy(wA).cuda() if amax_given else None
    p, s, Ad = nv.quantize_4over6(xd, A, err_mode="mae", e4m3_scale_bound=256, row_scaled=True)
    assert_bitwise(to_np(Ad), wA, "row amax (every row)")
    edge = 1 << 24
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(edge - 64, edge + 48),
                                     rng.integers(0, M, 4096)]))
    wp, ws = oracle.quantize_4over6(x[rows], wA[rows], err_mode="mae", bound=256.0)
    assert_bitwise(to_np(s)[rows], ws, "scales")
    assert_bitwise(to_np(p)[rows], wp, "codes")
