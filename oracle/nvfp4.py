"""NVFP4 quantize / dequantize / qdq / four-over-six / 2D, step by step
(oracle; test infrastructure only).

Notation (kept from the pages): x' is the input after the error-feedback add,
a is a block (or tile) absmax, A the global amax, S_enc / S_dec the global
encode / decode scales, sigma the fp32 block scale before its e4m3 cast, s the
decoded e4m3 scale, rho the encode reciprocal, v the scaled magnitude.

Inputs are float32 arrays (fp32 tensors) or uint16 arrays (bf16 bit
patterns), row-major [M, K] with K % 16 == 0.  The global element index of
(m, k) is (row_offset + m) * K + k; `row_offset` lets a caller run the oracle
on a slice of rows of a larger tensor, which is exact because rows are
independent on every path except the per-tensor amax (passed in).

Every float operation is one numpy float32 operation (IEEE RN, never fused).
"""
from __future__ import annotations

import numpy as np

from .formats import (
    E2M1_GRID,
    F32,
    FLT_MAX,
    bf16_bits_to_f32,
    e2m1_rtn_index,
    e2m1_sr_index,
    e4m3_decode,
    e4m3_encode,
    e4m3_encode_up,
    f32_to_bf16_bits,
)
from .rng import sr_u16

E4M3_MAX = F32(448.0)


def _to_f32(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    if x.dtype == np.float32:
        return x
    raise TypeError("input must be float32 values or uint16 bf16 bits")


def _check_k(K):
    if K % 16:
        raise ValueError("K must be a multiple of 16 (fp4-train, Requirements and limits)")


def _nan_drop_absmax(t, axis):
    """NaN-dropping max of |t| over `axis`; an all-NaN group gives 0
    (four-over-six pull request, CuTe DSL kernel Design: NaN-dropping block
    amaxes, all-NaN group -> amax 0)."""
    # every NaN counts as 0 before the max: np.fmax does not drop a
    # signalling NaN (the running max turns into a NaN there and restarts)
    a = np.abs(t)
    return np.max(np.where(np.isnan(a), F32(0.0), a), axis=axis, initial=F32(0.0)).astype(np.float32)


def _ef_add(x32, residual):
    """fp4-train, Method / API: with error feedback the carried residual is
    added into the next quantization: x' = x + r (one fp32 add)."""
    if residual is None:
        return x32
    r = np.asarray(residual, dtype=np.float32)
    if r.shape != x32.shape:
        raise ValueError("residual must be [M, K] float32")
    return x32 + r


def global_scales(A, bound):
    """S_enc = min(D / A, FLT_MAX) and S_dec = A / D with D = 6 * bound.

    Four-over-six pull request, What and CuTe DSL kernel Design: the global
    scale bound (448 standard, 256 for four-over-six) and true divisions for
    S_enc / S_dec.  The formula itself is not printed; D = 6 * bound is the
    reading under which the block holding A gets sigma = bound exactly the way
    the bound argument (256 * 1.5 = 384 < 448) needs, and under which the
    dequant error denominator is "6*bound".
    """
    D = F32(6.0 * bound)
    A = np.asarray(A, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        S_enc = np.fmin(D / A, FLT_MAX)
        S_dec = A / D
    return S_enc.astype(np.float32), S_dec.astype(np.float32), D


def _encode_reciprocal(s, S_dec):
    """rho = min(1 / (s * S_dec), FLT_MAX): four-over-six pull request, CuTe
    DSL kernel Design (the encode reciprocals).  Applied on every path: the
    fp4-train card's "divided by the decoded scale" is this reciprocal
    followed by a multiply.  s = 0 gives 1/0 = inf -> FLT_MAX."""
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return np.fmin(F32(1.0) / (s * S_dec), FLT_MAX).astype(np.float32)


def _encode(xp, rho, u16=None):
    """Element encode.  v = |x'| * rho; RTN (u16 None) or SR on the e2m1
    grid; sign bit from x' (so -0 keeps its sign); a NaN v encodes +6, code
    0x7 (four-over-six pull request, CuTe DSL kernel Design: NaN -> +6).
    Returns (code uint8, signed grid value float32)."""
    with np.errstate(invalid="ignore", over="ignore"):
        v = np.abs(xp) * rho
    nan = np.isnan(v)
    vv = np.where(nan, F32(0.0), v)
    idx = e2m1_rtn_index(vv) if u16 is None else e2m1_sr_index(vv, u16)
    idx = np.where(nan, 7, idx)
    neg = np.signbit(xp) & ~nan
    code = (neg.astype(np.uint8) << np.uint8(3)) | idx.astype(np.uint8)
    mag = E2M1_GRID[idx]
    val = np.where(neg, -mag, mag).astype(np.float32)
    return code, val


def pack_codes(codes) -> np.ndarray:
    """Two codes per byte along the last axis, even element in the low
    nibble (fp4-train, Method: codes pack two per byte; nibble order is this
    library's reading)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def code_values(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[(c & 7).astype(np.int64)]
    return np.where(c & 8, -mag, mag).astype(np.float32)


def _u16_grid(M, K, row_offset, seed, step):
    idx = (np.arange(M, dtype=np.int64)[:, None] + row_offset) * K + np.arange(K, dtype=np.int64)[None, :]
    return sr_u16(idx, seed, step)


def amax(x, residual=None, mode="tensor"):
    """Global amax A = NaN-dropping max of |x'| over the tensor ("tensor",
    a float32 scalar) or over each row ("row", shape [M]).  Four-over-six
    pull request, What: a scalar global_amax selects per-tensor scaling, a
    (rows,) vector the row-wise variant."""
    xp = _ef_add(_to_f32(x), residual)
    if mode == "tensor":
        return F32(_nan_drop_absmax(xp.reshape(-1), axis=0)) if xp.size else F32(0.0)
    if mode == "row":
        return _nan_drop_absmax(xp, axis=1)
    raise ValueError(mode)


def _standard_1x16(xp, global_amax, stochastic, seed, step, row_offset):
    """Shared steps of quantize / qdq on 1x16 blocks.  Returns codes [M,K],
    scale bytes [M,K/16], dequantized fp32 x_hat [M,K]."""
    M, K = xp.shape
    _check_k(K)
    blocks = xp.reshape(M, K // 16, 16)
    a = _nan_drop_absmax(blocks, axis=2)
    if global_amax is None:
        # fp4-train, Method: block scale = block_absmax / 6.
        S_dec = F32(1.0)
        sigma = a / F32(6.0)
    else:
        # Standard NVFP4 with a global scale (four-over-six pull request,
        # numeric details): sigma = block_amax * (S_enc * (1/6)), bound 448.
        S_enc, S_dec, _ = global_scales(global_amax, 448.0)
        with np.errstate(invalid="ignore", over="ignore"):
            sigma = a * (S_enc * (F32(1.0) / F32(6.0)))
    # NaN-dropping min for the 448 cap (CuTe DSL kernel Design).
    sigma = np.fmin(sigma, E4M3_MAX).astype(np.float32)
    sbyte = e4m3_encode(sigma)
    s = e4m3_decode(sbyte)
    rho = _encode_reciprocal(s, S_dec)
    u16 = None
    if stochastic:
        u16 = _u16_grid(M, K, row_offset, seed, step).reshape(M, K // 16, 16)
    codes, val = _encode(blocks, rho[..., None], u16)
    with np.errstate(invalid="ignore", over="ignore"):
        xhat = (val * s[..., None]) * S_dec
    return codes.reshape(M, K), sbyte, xhat.reshape(M, K).astype(np.float32)


def quantize(x, stochastic=False, residual=None, seed=0, step=0, global_amax=None, row_offset=0):
    """NVFP4 quantize on 1x16 blocks -> (packed [M, K/2] uint8, scales
    [M, K/16] uint8).

    fp4-train, API `quantize(x, stochastic, residual, seed, step)` and Method.
    With `residual` ([M, K] float32) it is error feedback: x' = x + r, and r is
    overwritten in place with x' - dequant(quant(x')) using the fp32 dequant
    value.  `global_amax` (optional float32 scalar A) adds the standard
    per-tensor second-level scale with bound 448.
    """
    xp = _ef_add(_to_f32(x), residual)
    codes, sbyte, xhat = _standard_1x16(xp, global_amax, stochastic, seed, step, row_offset)
    if residual is not None:
        residual[...] = xp - xhat
    return pack_codes(codes), sbyte


def dequantize(packed, scales, M, K, tile16=False, global_amax=None, scale_mode="none",
               bound=448.0, out="bf16"):
    """NVFP4 -> bf16 (default, as fp4-train's API) or fp32.

    x_hat = (val * s) * S_dec: val * s is exact; the S_dec multiply is one
    rounding (exact when there is no global scale, S_dec = 1), then bf16 RNE.
    `scales` is [M, K/16] (1x16 blocks) or [M/16, K/16] (tile16).  The global
    scale is none, one amax for the tensor, or one per row ("row"), with the
    bound the producer used.
    """
    _check_k(K)
    codes = unpack_codes(np.asarray(packed).reshape(M, K // 2))
    val = code_values(codes)
    s = e4m3_decode(np.asarray(scales))
    if tile16:
        s_el = np.repeat(np.repeat(s.reshape(M // 16, K // 16), 16, axis=0), 16, axis=1)
    else:
        s_el = np.repeat(s.reshape(M, K // 16), 16, axis=1)
    if scale_mode == "none":
        S_dec = F32(1.0)
    else:
        _, S_dec, _ = global_scales(global_amax, bound)
        if scale_mode == "row":
            S_dec = S_dec.reshape(M, 1)
    with np.errstate(invalid="ignore", over="ignore"):
        xhat = ((val * s_el) * S_dec).astype(np.float32)
    return f32_to_bf16_bits(xhat) if out == "bf16" else xhat


def qdq(x, stochastic=False, residual=None, seed=0, step=0, global_amax=None, out="bf16",
        row_offset=0):
    """Quantize then dequantize, "the value the tensor cores use" (fp4-train,
    API).  Returns (out, packed, scales); out is bf16 bits or fp32.  With a
    residual this is the error-feedback step; r uses the fp32 dequant value,
    before the bf16 rounding of the output."""
    xp = _ef_add(_to_f32(x), residual)
    codes, sbyte, xhat = _standard_1x16(xp, global_amax, stochastic, seed, step, row_offset)
    if residual is not None:
        residual[...] = xp - xhat
    o = f32_to_bf16_bits(xhat) if out == "bf16" else xhat
    return o, pack_codes(codes), sbyte


def _tree16(e):
    """The exact width-16 reduction of 16 row errors (last axis) given in the
    four-over-six pull request (CuTe DSL kernel Design)."""
    g = [e[..., i] for i in range(16)]
    left = ((g[0] + g[8]) + (g[4] + g[12])) + ((g[2] + g[10]) + (g[6] + g[14]))
    right = ((g[1] + g[9]) + (g[5] + g[13])) + ((g[3] + g[11]) + (g[7] + g[15]))
    return left + right


def quantize_4over6(x, global_amax, err_mode="mae", bound=256.0, block="1x16"):
    """Four-over-six NVFP4 quantize -> (packed [M, K/2], scales).

    Four-over-six pull request, What: every block is encoded twice - map-to-6
    and map-to-4, whose scale is expanded by 1.5x - and the candidate with the
    lower dequantization error (MAE or MSE) is stored; ties select map-to-6.
    Numeric details: sigma6 = (block_amax / 6) * S_enc; true fp32 divisions
    on the selection path.  CuTe DSL kernel Design: encode reciprocals
    min(1/(s * S_dec), FLT_MAX); the dequant error uses the denominator
    6 * bound; NaN-dropping 448 caps; per-16 errors summed strictly in element
    order 0..15; 16x16 tiles combine their 16 row errors with the exact
    width-16 tree; strict err4 < err6 (ties and NaN pick map-to-6).  No
    stochastic rounding (What).

    global_amax: float32 scalar (per tensor) or [M] vector (row-wise; 1x16
    only).  Readings: sigma4 = sigma6 * 1.5 on the fp32 value before the e4m3
    cast; the error dequant is d = ((val * s) * A) / D, D = 6 * bound.
    Returns scales [M, K/16] for 1x16 and [M/16, K/16] for 16x16.
    """
    xp = _to_f32(x)
    M, K = xp.shape
    _check_k(K)
    A = np.asarray(global_amax, dtype=np.float32)
    row = A.ndim == 1
    if row and block != "1x16":
        raise ValueError("row-wise global amax is 1x16 only")
    S_enc, S_dec, D = global_scales(A, bound)
    if block == "1x16":
        xb = xp.reshape(M, K // 16, 16)  # [M, nb, 16]
        a = _nan_drop_absmax(xb, axis=2)
        bshape = (M, 1) if row else ()
    elif block == "16x16":
        if M % 16:
            raise ValueError("16x16 blocks need M % 16 == 0")
        xb = xp.reshape(M // 16, 16, K // 16, 16).transpose(0, 2, 1, 3)  # [ti, tj, r, c]
        a = _nan_drop_absmax(xb, axis=(2, 3))
        bshape = ()
    else:
        raise ValueError(block)
    Ab = A.reshape(bshape) if row else A
    S_enc_b = S_enc.reshape(bshape) if row else S_enc
    S_dec_b = S_dec.reshape(bshape) if row else S_dec
    with np.errstate(invalid="ignore", over="ignore"):
        sig6 = (a / F32(6.0)) * S_enc_b
        sig4 = sig6 * F32(1.5)
    cand = []
    for sig in (sig6, sig4):
        sig = np.fmin(sig, E4M3_MAX).astype(np.float32)
        sbyte = e4m3_encode(sig)
        s = e4m3_decode(sbyte)
        rho = _encode_reciprocal(s, S_dec_b)
        if block == "1x16":
            codes, val = _encode(xb, rho[..., None], None)
            s_el = s[..., None]
            A_el = Ab[..., None] if row else Ab
        else:
            codes, val = _encode(xb, rho[..., None, None], None)
            s_el = s[..., None, None]
            A_el = Ab
        with np.errstate(invalid="ignore", over="ignore"):
            d = ((val * s_el) * A_el) / D
            t = xb - d
            e = np.abs(t) if err_mode == "mae" else t * t
        if block == "1x16":
            E = e[..., 0]
            for i in range(1, 16):
                E = E + e[..., i]
        else:
            er = e[..., 0]
            for i in range(1, 16):
                er = er + e[..., i]          # per tile row, element order
            E = _tree16(er)                  # 16 row errors -> tile error
        cand.append((codes, sbyte, E))
    (c6, b6, E6), (c4, b4, E4) = cand
    pick4 = E4 < E6
    if block == "1x16":
        codes = np.where(pick4[..., None], c4, c6).reshape(M, K)
        sbyte = np.where(pick4, b4, b6).astype(np.uint8)
    else:
        codes_t = np.where(pick4[..., None, None], c4, c6)  # [ti, tj, r, c]
        codes = codes_t.transpose(0, 2, 1, 3).reshape(M, K)
        sbyte = np.where(pick4, b4, b6).astype(np.uint8)
    return pack_codes(codes), sbyte


def quantize_4over6_2d(x, global_amax, err_mode="mae", bound=256.0):
    """Four-over-six on transposition-invariant 16x16 tiles (per-tensor
    global amax) -> (packed_row [M, K/2], packed_col [K, M/2], tile_scales
    [M/16, K/16]).  The tile's candidate choice uses the 16 per-row
    sequential errors combined by the exact width-16 tree (four-over-six
    pull request, CuTe DSL kernel Design); rowwise and columnwise outputs are
    the same codes, so they share the tile scale (transposition-invariant 2D
    paper, abstract)."""
    packed, scales = quantize_4over6(x, global_amax, err_mode=err_mode, bound=bound, block="16x16")
    xp = _to_f32(x)
    M, K = xp.shape
    codes = unpack_codes(packed).reshape(M, K)
    return packed, pack_codes(codes.T), scales


def quantize_rowcol(x, global_amax, four_over_six=False, err_mode="mae", bound=448.0):
    """Rowwise and columnwise 1x16 quantization of the same tensor in one
    call -> (packed_row [M, K/2], scales_row [M, K/16], packed_col [K, M/2],
    scales_col [K, M/16]).  The columnwise outputs are the rowwise
    quantization of X^T (blocks of 16 consecutive rows of one column), as the
    backward-pass operands need (four-over-six pull request, What: backward
    against saved columnwise codes; Follow-up fusions: a fused row + col
    kernel instead of x.t().contiguous()).  Round-to-nearest with one
    per-tensor global amax: the standard path (sigma = a * (S_enc * (1/6)),
    bound 448) or four-over-six (bound 256 or 448)."""
    xp = _to_f32(x)
    M, K = xp.shape
    if M % 16:
        raise ValueError("columnwise 1x16 blocks need M % 16 == 0")
    A = np.float32(global_amax)
    xt = np.ascontiguousarray(xp.T)
    if four_over_six:
        pr, sr = quantize_4over6(xp, A, err_mode=err_mode, bound=bound)
        pc, scol = quantize_4over6(xt, A, err_mode=err_mode, bound=bound)
    else:
        if bound != 448.0:
            raise ValueError("the standard path uses bound 448")
        pr, sr = quantize(xp, global_amax=A)
        pc, scol = quantize(xt, global_amax=A)
    return pr, sr, pc, scol


def quantize_2d(x, stochastic=False, seed=0, step=0, global_amax=None, row_offset=0,
                truncation_free=False):
    """Transposition-invariant 2D NVFP4: one e4m3 scale per 16x16 tile,
    shared by X and X^T ("Stable FP4 Training via Transposition-Invariant
    Block Quantization", abstract), optionally with stochastic rounding.

    Every element is encoded once (RNG index = its row-major index in X).
    Returns (packed_row [M, K/2], packed_col [K, M/2], tile_scales
    [M/16, K/16]); packed_col is the same codes transposed, so it is the
    rowwise packing of Q(X)^T.  The block scale follows the standard path:
    a/6 without a global scale, a * (S_enc * (1/6)) with one (bound 448).
    `row_offset` must be a multiple of 16.
    """
    xp = _to_f32(x)
    M, K = xp.shape
    _check_k(K)
    if M % 16 or row_offset % 16:
        raise ValueError("2D blocks need M % 16 == 0")
    xt = xp.reshape(M // 16, 16, K // 16, 16)
    a = _nan_drop_absmax(xt, axis=(1, 3))  # [M/16, K/16]
    if global_amax is None:
        S_dec = F32(1.0)
        sigma = a / F32(6.0)
    else:
        S_enc, S_dec, _ = global_scales(global_amax, 448.0)
        with np.errstate(invalid="ignore", over="ignore"):
            sigma = a * (S_enc * (F32(1.0) / F32(6.0)))
    sigma = np.fmin(sigma, E4M3_MAX).astype(np.float32)
    sbyte = e4m3_encode_up(sigma) if truncation_free else e4m3_encode(sigma)
    s = e4m3_decode(sbyte)
    rho = _encode_reciprocal(s, S_dec)
    rho_el = np.repeat(np.repeat(rho, 16, axis=0), 16, axis=1)
    u16 = _u16_grid(M, K, row_offset, seed, step) if stochastic else None
    codes, _ = _encode(xp, rho_el, u16)
    return pack_codes(codes), pack_codes(codes.T), sbyte
