"""ctypes loader for libnvfp4.so (the HIP kernels behind the C ABI declared in
include/nvfp4.h).  Loading fails loudly when the library has not been built:
there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

# status codes (nvfp4_status)
OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_ARG, E_RANGE, E_HIP = range(8)
# enums
F32, BF16 = 0, 1
RTN, SR = 0, 1
MAE, MSE = 0, 1
SCALE_NONE, SCALE_TENSOR, SCALE_ROW = 0, 1, 2

_c = ctypes
_vp, _i64, _u32, _i32, _f32, _sz = _c.c_void_p, _c.c_int64, _c.c_uint32, _c.c_int, _c.c_float, _c.c_size_t

# name -> (restype, argtypes); mirrors include/nvfp4.h
SIGNATURES = {
    "nvfp4_status_str": (_c.c_char_p, [_i32]),
    "nvfp4_amax_workspace_bytes": (_sz, [_i64, _i64]),
    "nvfp4_amax": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp]),
    "nvfp4_amax_noalloc": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _vp, _vp]),
    "nvfp4_quantize": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _u32, _u32, _vp, _vp, _vp]),
    "nvfp4_dequantize": (_i32, [_vp, _vp, _i64, _i64, _i32, _vp, _i32, _f32, _vp, _i32, _vp]),
    "nvfp4_qdq": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _u32, _u32, _vp, _i32, _vp, _vp, _vp]),
    "nvfp4_quantize_4over6": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _i32, _f32, _vp, _vp, _vp]),
    "nvfp4_quantize_2d": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _u32, _u32, _i32, _vp, _vp, _vp, _vp]),
    "nvfp4_quantize_rowcol": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp]),
    "nvfp4_quantize_4over6_2d": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _f32, _vp, _vp, _vp, _vp]),
    "nvfp4_selftest_scan": (_i32, [_i32, _u32, _c.c_uint64, _c.c_uint64, _i32, _vp, _vp]),
    "nvfp4_selftest_launch_plan": (_i32, [_i32, _i64, _i64, _i32, _i32, _vp]),
}


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m fp4_block_quantization_nvfp4_amd.build`"
            )
        dll = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(dll, name)
            fn.restype = res
            fn.argtypes = args
        _lib = dll
    return _lib


def status_str(status: int) -> str:
    return lib().nvfp4_status_str(status).decode()


def check(status: int, what: str) -> None:
    if status != OK:
        raise NVFP4Error(status, what)
