"""Graph capture of the allocation-free path, through the C ABI: the
per-tensor amax into the library's own scratch array (nvfp4_amax_noalloc),
then four-over-six 1x16 and 2D + SR quantize with that amax, all captured in
one HIP graph by a caller that allocates nothing inside the capture.  The
graph is replayed four times; before each replay the captured input buffer
gets new contents, and between replays eager calls run on other buffers
(one of them overwrites the shared scratch array).  Every replay's amax,
codes and scales must equal eager calls on the same input bit for bit, and
the four-over-six rows sampled against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import fp4_block_quantization_nvfp4_amd as nv
from fp4_block_quantization_nvfp4_amd import _lib as L
from tests.gpu_util import assert_bitwise, need_gpu, to_dev, to_np, wide_input

pytestmark = pytest.mark.gpu

M, K = 2048, 7168
SEED, STEP = 11, 3


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _captured_calls(lib, st, x, A, p46, s46, p2r, p2c, t2):
    L.check(lib.nvfp4_amax_noalloc(x.data_ptr(), L.BF16, M, K, None, L.SCALE_TENSOR, A.data_ptr(), st),
            "nvfp4_amax_noalloc")
    L.check(lib.nvfp4_quantize_4over6(x.data_ptr(), L.BF16, M, K, A.data_ptr(), L.SCALE_TENSOR, 1, L.MAE,
                                      256.0, p46.data_ptr(), s46.data_ptr(), st), "nvfp4_quantize_4over6")
    L.check(lib.nvfp4_quantize_2d(x.data_ptr(), L.BF16, M, K, A.data_ptr(), L.SR, SEED, STEP, 0,
                                  p2r.data_ptr(), p2c.data_ptr(), t2.data_ptr(), st), "nvfp4_quantize_2d")


def test_graph_replays_of_noalloc_amax_and_quantize():
    lib = L.lib()
    inputs = [wide_input(300 + i, M, K, bf16=True) for i in range(5)]
    dev = lambda shape: torch.empty(shape, dtype=torch.uint8, device="cuda")
    x = to_dev(inputs[0]).clone()
    A = torch.zeros(1, dtype=torch.float32, device="cuda")
    p46, s46 = dev((M, K // 2)), dev((M, K // 16))
    p2r, p2c, t2 = dev((M, K // 2)), dev((K, M // 2)), dev((M // 16, K // 16))
    # eager first call: the library finds its scratch array's address here
    _captured_calls(lib, torch.cuda.current_stream().cuda_stream, x, A, p46, s46, p2r, p2c, t2)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        _captured_calls(lib, torch.cuda.current_stream().cuda_stream, x, A, p46, s46, p2r, p2c, t2)
    torch.cuda.synchronize()

    other = to_dev(wide_input(399, 512, 1040, bf16=True))
    A_other = torch.empty(1, dtype=torch.float32, device="cuda")
    rows = np.array([0, 1, 777, M - 1])
    for i in range(1, 5):
        x.copy_(to_dev(inputs[i]))
        g.replay()
        torch.cuda.synchronize()
        got = [to_np(t).copy() for t in (A, p46, s46, p2r, p2c, t2)]
        # eager work between replays: another tensor through the same scratch array
        st = torch.cuda.current_stream().cuda_stream
        L.check(lib.nvfp4_amax_noalloc(other.data_ptr(), L.BF16, 512, 1040, None, L.SCALE_TENSOR,
                                       A_other.data_ptr(), st), "nvfp4_amax_noalloc")
        torch.cuda.synchronize()
        assert_bitwise(to_np(A_other), np.atleast_1d(oracle.amax(to_np(other))), f"replay {i}: other amax")
        # eager reference on the same input, separate buffers
        xe = to_dev(inputs[i])
        Ae = nv.amax(xe)
        pe, se, _ = nv.quantize_4over6(xe, Ae, err_mode="mae", e4m3_scale_bound=256)
        re, ce, te = nv.quantize_2d(xe, global_amax=Ae, stochastic=True, seed=SEED, step=STEP)
        want = [to_np(t) for t in (Ae, pe, se, re, ce, te)]
        for name, a, b in zip(("amax", "4over6 codes", "4over6 scales", "2d row codes", "2d column codes",
                               "2d tile scales"), got, want):
            assert_bitwise(a, b, f"replay {i}: {name}")
        wA = np.float32(oracle.amax(inputs[i]))
        assert_bitwise(got[0], np.atleast_1d(wA), f"replay {i}: amax vs oracle")
        wp, ws = oracle.quantize_4over6(inputs[i][rows], wA, err_mode="mae", bound=256.0)
        assert_bitwise(got[1][rows], wp, f"replay {i}: 4over6 codes vs oracle")
        assert_bitwise(got[2][rows], ws, f"replay {i}: 4over6 scales vs oracle")
