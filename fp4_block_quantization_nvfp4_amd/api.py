"""Python binding of libnvfp4: argument marshalling only.

Every function takes and returns torch tensors on the current HIP device,
allocates its outputs with torch, and calls one or more C-ABI entry points on
torch's current stream.  All arithmetic runs in the HIP kernels; there is no
CPU path.  Names follow the pages: `quantize / dequantize / qdq /
ErrorFeedback` as in the fp4-train card's API, `quantize_4over6` as the
four-over-six pull request's `four_over_six_quantize`, and `quantize_2d` for
the transposition-invariant 16x16 variant.
"""
from __future__ import annotations

import torch

from . import _lib as L

_DT = {torch.float32: L.F32, torch.bfloat16: L.BF16}


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_input(x: torch.Tensor, what: str):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{what}: a device tensor is required (no CPU path)")
    if x.dim() != 2:
        raise ValueError(f"{what}: a 2-D [M, K] tensor is required")
    if x.dtype not in _DT:
        raise ValueError(f"{what}: float32 or bfloat16 input required")
    if not x.is_contiguous():
        raise ValueError(f"{what}: input must be contiguous")
    return x.shape[0], x.shape[1]


def _check_residual(residual, x):
    if residual is None:
        return None
    if residual.dtype != torch.float32 or residual.shape != x.shape or not residual.is_contiguous() \
            or residual.device != x.device:
        raise ValueError("residual must be a contiguous float32 [M, K] tensor on x's device")
    return residual


def _amax_arg(global_amax, x, rows):
    if global_amax is None:
        return None
    if not isinstance(global_amax, torch.Tensor):
        global_amax = torch.tensor([float(global_amax)], dtype=torch.float32, device=x.device)
    g = global_amax.reshape(-1)
    if g.dtype != torch.float32 or g.device != x.device:
        raise ValueError("global_amax must be float32 on x's device")
    if g.numel() not in ((rows,) if rows is not None else (1,)):
        raise ValueError("global_amax has the wrong number of elements")
    return g.contiguous()


def amax(x: torch.Tensor, residual: torch.Tensor | None = None, mode: str = "tensor") -> torch.Tensor:
    """NaN-dropping max of |x + residual| per tensor (shape [1]) or per row ([M])."""
    M, K = _check_input(x, "amax")
    residual = _check_residual(residual, x)
    m = {"tensor": L.SCALE_TENSOR, "row": L.SCALE_ROW}[mode]
    out = torch.empty(1 if m == L.SCALE_TENSOR else M, dtype=torch.float32, device=x.device)
    nws = L.lib().nvfp4_amax_workspace_bytes(M, K)
    ws = torch.empty(max(nws, 4), dtype=torch.uint8, device=x.device)
    L.check(L.lib().nvfp4_amax(_ptr(x), _DT[x.dtype], M, K, _ptr(residual), m, _ptr(out),
                               _ptr(ws), ws.numel(), _stream()), "nvfp4_amax")
    return out


def _resolve_global(global_amax, x, residual=None):
    if isinstance(global_amax, str):
        if global_amax != "compute":
            raise ValueError("global_amax must be None, 'compute', a float or a tensor")
        return amax(x, residual, "tensor")
    return _amax_arg(global_amax, x, None)


def quantize(x, stochastic=False, residual=None, seed=0, step=0, global_amax=None):
    """NVFP4 quantize -> (packed uint8 [M, K/2], scale uint8 [M, K/16]).

    residual: optional float32 [M, K] error-feedback residual, updated in
    place.  global_amax: None, 'compute', a float or a float32 tensor [1].
    """
    M, K = _check_input(x, "quantize")
    residual = _check_residual(residual, x)
    ga = _resolve_global(global_amax, x, residual)
    packed = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scale = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    L.check(L.lib().nvfp4_quantize(_ptr(x), _DT[x.dtype], M, K, _ptr(residual), _ptr(ga),
                                   L.SR if stochastic else L.RTN, seed & 0xFFFFFFFF,
                                   step & 0xFFFFFFFF, _ptr(packed), _ptr(scale), _stream()),
            "nvfp4_quantize")
    return packed, scale


def dequantize(packed, scale, M, K, *, tile16=False, global_amax=None, row_scaled=False,
               bound=448.0, out_dtype=torch.bfloat16):
    """NVFP4 -> out_dtype [M, K].  `global_amax`/`row_scaled`/`bound` name the
    producer's second-level scale."""
    if not packed.is_cuda or not scale.is_cuda:
        raise ValueError("dequantize: device tensors required")
    if packed.dtype != torch.uint8 or scale.dtype != torch.uint8:
        raise ValueError("dequantize: uint8 codes and scales required")
    nbr = (M // 16) if tile16 else M
    if packed.numel() != M * K // 2 or scale.numel() != nbr * (K // 16):
        raise ValueError("dequantize: packed/scale sizes do not match M, K")
    mode = L.SCALE_NONE
    ga = None
    if global_amax is not None:
        mode = L.SCALE_ROW if row_scaled else L.SCALE_TENSOR
        ga = _amax_arg(global_amax, packed, M if row_scaled else None)
    out = torch.empty((M, K), dtype=out_dtype, device=packed.device)
    L.check(L.lib().nvfp4_dequantize(_ptr(packed.contiguous()), _ptr(scale.contiguous()), M, K,
                                     int(tile16), _ptr(ga), mode, float(bound), _ptr(out),
                                     _DT[out_dtype], _stream()), "nvfp4_dequantize")
    return out


def qdq(x, stochastic=False, residual=None, seed=0, step=0, global_amax=None,
        out_dtype=torch.bfloat16, return_codes=False, out=None):
    """Quantize then dequantize in one kernel -> out [M, K] (bf16 by default);
    with return_codes also (packed, scale)."""
    M, K = _check_input(x, "qdq")
    residual = _check_residual(residual, x)
    ga = _resolve_global(global_amax, x, residual)
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=x.device)
    elif out.shape != x.shape or out.dtype not in _DT or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, K] float32/bfloat16 tensor")
    packed = scale = None
    if return_codes:
        packed = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        scale = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    L.check(L.lib().nvfp4_qdq(_ptr(x), _DT[x.dtype], M, K, _ptr(residual), _ptr(ga),
                              L.SR if stochastic else L.RTN, seed & 0xFFFFFFFF,
                              step & 0xFFFFFFFF, _ptr(out), _DT[out.dtype], _ptr(packed),
                              _ptr(scale), _stream()), "nvfp4_qdq")
    return (out, packed, scale) if return_codes else out


def quantize_4over6(x, global_amax=None, *, err_mode="mae", e4m3_scale_bound=256,
                    row_scaled=None):
    """Four-over-six quantize on 1x16 blocks -> (packed, scale, global_amax).

    global_amax: a float32 scalar tensor (per-tensor scaling), a [M] vector
    (row-wise scaling), or None with row_scaled=True to compute the per-row
    amax inside the same kernel (returned as the third output).
    """
    M, K = _check_input(x, "quantize_4over6")
    err = {"mae": L.MAE, "mse": L.MSE}[err_mode]
    if global_amax is None:
        if not row_scaled:
            global_amax = amax(x, mode="tensor")
            mode, given = L.SCALE_TENSOR, 1
        else:
            global_amax = torch.empty(M, dtype=torch.float32, device=x.device)
            mode, given = L.SCALE_ROW, 0
    else:
        g = global_amax.reshape(-1) if isinstance(global_amax, torch.Tensor) else global_amax
        rows = isinstance(g, torch.Tensor) and g.numel() == M and (row_scaled or (M != 1))
        if row_scaled is False:
            rows = False
        global_amax = _amax_arg(g, x, M if rows else None)
        mode, given = (L.SCALE_ROW if rows else L.SCALE_TENSOR), 1
    packed = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scale = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    L.check(L.lib().nvfp4_quantize_4over6(_ptr(x), _DT[x.dtype], M, K, _ptr(global_amax), mode,
                                          given, err, float(e4m3_scale_bound), _ptr(packed),
                                          _ptr(scale), _stream()), "nvfp4_quantize_4over6")
    return packed, scale, global_amax


def quantize_2d(x, global_amax=None, stochastic=False, seed=0, step=0, columnwise=True,
                truncation_free=False):
    """Transposition-invariant 16x16 quantize -> (packed_row [M, K/2],
    packed_col [K, M/2] or None, tile_scales [M/16, K/16]).  truncation_free
    rounds each tile scale up instead of to nearest."""
    M, K = _check_input(x, "quantize_2d")
    ga = _resolve_global(global_amax, x)
    packed_row = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    packed_col = torch.empty((K, M // 2), dtype=torch.uint8, device=x.device) if columnwise else None
    tiles = torch.empty((M // 16, K // 16), dtype=torch.uint8, device=x.device)
    L.check(L.lib().nvfp4_quantize_2d(_ptr(x), _DT[x.dtype], M, K, _ptr(ga),
                                      L.SR if stochastic else L.RTN, seed & 0xFFFFFFFF,
                                      step & 0xFFFFFFFF, int(bool(truncation_free)),
                                      _ptr(packed_row), _ptr(packed_col), _ptr(tiles), _stream()),
            "nvfp4_quantize_2d")
    return packed_row, packed_col, tiles


def quantize_rowcol(x, global_amax="compute", *, four_over_six=False, err_mode="mae",
                    e4m3_scale_bound=None):
    """Rowwise and columnwise 1x16 NVFP4 of x in one pass (RTN, one global
    amax) -> (packed_row [M, K/2], scales_row [M, K/16], packed_col [K, M/2],
    scales_col [K, M/16]); the columnwise pair is the quantization of x^T.
    Standard encode (bound 448) or four-over-six (bound 256 by default)."""
    M, K = _check_input(x, "quantize_rowcol")
    ga = _resolve_global(global_amax, x)
    if ga is None:
        raise ValueError("quantize_rowcol needs a global amax ('compute', a float or a tensor)")
    bound = e4m3_scale_bound if e4m3_scale_bound is not None else (256 if four_over_six else 448)
    err = {"mae": L.MAE, "mse": L.MSE}[err_mode]
    dev = x.device
    pr = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sr = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    pc = torch.empty((K, M // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((K, M // 16), dtype=torch.uint8, device=dev)
    L.check(L.lib().nvfp4_quantize_rowcol(_ptr(x), _DT[x.dtype], M, K, _ptr(ga), int(bool(four_over_six)),
                                          err, float(bound), _ptr(pr), _ptr(sr), _ptr(pc), _ptr(sc),
                                          _stream()), "nvfp4_quantize_rowcol")
    return pr, sr, pc, sc


def quantize_4over6_2d(x, global_amax="compute", *, err_mode="mae", e4m3_scale_bound=256,
                       columnwise=True):
    """Four-over-six on 16x16 tiles (one global amax) -> (packed_row [M, K/2],
    packed_col [K, M/2] or None, tile_scales [M/16, K/16])."""
    M, K = _check_input(x, "quantize_4over6_2d")
    ga = _resolve_global(global_amax, x)
    if ga is None:
        raise ValueError("quantize_4over6_2d needs a global amax ('compute', a float or a tensor)")
    err = {"mae": L.MAE, "mse": L.MSE}[err_mode]
    dev = x.device
    pr = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    pc = torch.empty((K, M // 2), dtype=torch.uint8, device=dev) if columnwise else None
    ts = torch.empty((M // 16, K // 16), dtype=torch.uint8, device=dev)
    L.check(L.lib().nvfp4_quantize_4over6_2d(_ptr(x), _DT[x.dtype], M, K, _ptr(ga), err,
                                             float(e4m3_scale_bound), _ptr(pr), _ptr(pc), _ptr(ts),
                                             _stream()), "nvfp4_quantize_4over6_2d")
    return pr, pc, ts


class ErrorFeedback:
    """Per-tensor error-feedback state for weights stored in NVFP4 (fp4-train,
    API `ErrorFeedback`): `qdq(name, x, step)` adds the carried residual,
    quantizes, dequantizes, and banks the new residual for `name`."""

    def __init__(self, stochastic: bool = False, seed: int = 0):
        self.stochastic = stochastic
        self.seed = seed
        self.residuals: dict[str, torch.Tensor] = {}

    def qdq(self, name: str, x: torch.Tensor, step: int = 0, out_dtype=torch.bfloat16):
        r = self.residuals.get(name)
        if r is None or r.shape != x.shape:
            r = torch.zeros(x.shape, dtype=torch.float32, device=x.device)
            self.residuals[name] = r
        return qdq(x.contiguous(), self.stochastic, r, self.seed, step, out_dtype=out_dtype)

    def state_dict(self):
        return {k: v.clone() for k, v in self.residuals.items()}

    def load_state_dict(self, state):
        self.residuals = {k: v.clone() for k, v in state.items()}
