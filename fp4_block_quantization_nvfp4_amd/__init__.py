"""NVFP4 block quantization for AMD Instinct MI355X (CDNA4, gfx950).

The work is done by hand-written HIP kernels in libnvfp4.so behind a C ABI
(include/nvfp4.h); this package is its thin torch-facing binding.
"""
from ._lib import NVFP4Error, lib  # noqa: F401
from .api import (  # noqa: F401
    ErrorFeedback,
    amax,
    dequantize,
    qdq,
    quantize,
    quantize_2d,
    quantize_4over6_2d,
    quantize_rowcol,
    quantize_4over6,
)
