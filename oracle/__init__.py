"""CPU oracle for NVFP4 block quantization.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference that the
HIP library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path (the HIP library
and its Python binding) never does, and this package never imports the
product.  The two share no code: the only common module is the seeded input
generator (`workloads`), which holds none of the method's arithmetic.

Arithmetic is numpy float32: every `+ - * /` is one IEEE binary32 operation
rounded to nearest-even and never fused; `np.fmin` drops a (quiet) NaN, and
the NaN-dropping amax maps every NaN of the input, signalling ones included,
to 0 before its max.  bf16
values are handled as uint16 bit patterns.  Computation is vectorised over
independent blocks only; within a block every step is taken in the order the
pages give it.

Sources (the pages this follows):

* "fp4-train" kernel card - sections Method, API, Correctness, Requirements
  and limits: e2m1 grid, e4m3 block scale = block absmax / 6, stochastic
  rounding from a counter-based (seed, step, global-index) generator, error
  feedback, dequantize, qdq, zero-scale blocks.
* "Add NVFP4 four-over-six (row-wise) quantization to the training prototype"
  (torchao pull request) - sections What, the two numeric details, CuTe DSL
  kernel design, bitwise validation: global scale bound, four-over-six
  candidates and selection, scale associations, reciprocal rule, NaN rules,
  error accumulation order.
* "Stable FP4 Training via Transposition-Invariant Block Quantization" -
  abstract: 16x16 2D blocks whose scale is shared by X and X^T, combined with
  stochastic rounding.

Parity status of each function is stated in its docstring.  The random-number
generator's exact bits are a choice the pages leave open ("counter-based
(seed, step, global-index)"): its bits are parity unpinned against the pages
and pinned only by statistics and structure (tests/test_oracle_rng.py).
"""
from .formats import (  # noqa: F401
    E2M1_GRID,
    E4M3_VALUES,
    FLT_MAX,
    bf16_bits_to_f32,
    e2m1_rtn_index,
    e2m1_sr_index,
    e4m3_decode,
    e4m3_encode,
    e4m3_encode_up,
    f32_to_bf16_bits,
)
from .rng import pcg_hash, rng_key, sr_u16  # noqa: F401
from .nvfp4 import (  # noqa: F401
    amax,
    dequantize,
    qdq,
    quantize,
    quantize_2d,
    quantize_4over6,
    quantize_4over6_2d,
    quantize_rowcol,
    unpack_codes,
)
