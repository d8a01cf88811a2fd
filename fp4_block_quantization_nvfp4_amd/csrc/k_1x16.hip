// 1x16-block NVFP4 quantize / qdq (with optional error feedback and
// stochastic rounding) and dequantize.
//
// "fp4-train" kernel card, Method: each 16-element block gets the scale
// block_absmax / 6 encoded to e4m3; elements are divided by the decoded scale
// (an encode reciprocal here) and rounded to the e2m1 grid, to nearest or
// stochastically from a counter-based (seed, step, global-index) generator;
// with error feedback the residual x - dequant(quantize(x)) is carried into
// the next call.  With a global amax the standard NVFP4 two-level scale is
// used (four-over-six pull request, numeric details: block_amax *
// (S_enc * (1/6)), bound 448).
//
// Layout and mapping: blocks never straddle rows (K % 16 == 0), so the
// [M, K] tensor is a flat run of M*K/16 blocks and block b owns codes
// bytes [8b, 8b+8), scale byte b and elements [16b, 16b+16).  One lane owns
// one block: it reads 32 B (bf16) or 64 B (fp32) with 128-bit loads, reduces
// the block amax in registers, and writes 8 B of codes with one 64-bit store,
// so a wave covers 64 consecutive blocks and every access of a wave is one
// contiguous span.  The work is pure streaming (HBM-bound): no LDS, no MFMA.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

constexpr int kThreads = 256;

template <typename InT, bool HAS_RES, bool SR, bool GLOBAL, int OUT, bool CODES>
__global__ __launch_bounds__(kThreads) void k_quant1x16(
    const InT* x, float* __restrict__ residual, const float* __restrict__ global_amax,
    uint32_t key, int64_t nblk, uint8_t* __restrict__ packed, uint8_t* __restrict__ scales,
    void* out) {
  const int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= nblk) return;

  float S_dec = 1.0f, mul = 0.0f;
  if (GLOBAL) {
    float S_enc;
    global_scales(global_amax[0], 2688.0f, S_enc, S_dec);
    mul = S_enc * (1.0f / 6.0f);
  }

  float xv[16];
  load16(x + blk * 16, xv);
  if (HAS_RES) {
    float r[16];
    load16(residual + blk * 16, r);
#pragma unroll
    for (int i = 0; i < 16; ++i) xv[i] = xv[i] + r[i];
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xv[i]));

  float sigma = GLOBAL ? a * mul : a / 6.0f;
  sigma = fminf(sigma, kE4m3Max);
  const uint32_t sc = e4m3_encode(sigma);
  const float s = e4m3_decode(sc);
  const float rho = encode_reciprocal(s, S_dec);

  uint32_t w[8];
  if (SR) {
    const uint32_t p0 = (uint32_t)(blk * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = pcg_hash((p0 + j) ^ key);
  }

  uint32_t c0 = 0, c1 = 0;
  float xh[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = fabsf(xv[i]) * rho;
    float q;
    uint32_t mag;
    if (SR) mag = e2m1_sr(v, (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu, q);
    else mag = e2m1_rtn(v, q);
    const bool nan_v = (v != v);
    const uint32_t neg = nan_v ? 0u : (f2bits(xv[i]) >> 31);
    const uint32_t code = mag | (neg << 3);
    if (i < 8) c0 |= code << (4 * i);
    else c1 |= code << (4 * (i - 8));
    const float val = neg ? -q : q;
    xh[i] = (val * s) * S_dec;
  }

  if (CODES) {
    reinterpret_cast<uint2*>(packed)[blk] = make_uint2(c0, c1);
    scales[blk] = (uint8_t)sc;
  }
  if (HAS_RES) {
    float r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = xv[i] - xh[i];
    store16(residual + blk * 16, r);
  }
  if (OUT == 1) store16_bf16(reinterpret_cast<uint16_t*>(out) + blk * 16, xh);
  if (OUT == 2) store16(reinterpret_cast<float*>(out) + blk * 16, xh);
}

template <typename InT, bool HAS_RES, bool SR, bool GLOBAL>
static int dispatch_out(const InT* x, float* res, const float* ga, uint32_t key, int64_t nblk,
                        uint8_t* packed, uint8_t* scales, void* out, int out_kind,
                        hipStream_t st) {
  const dim3 grid((unsigned)((nblk + kThreads - 1) / kThreads)), block(kThreads);
  const bool codes = packed != nullptr;
  if (out_kind == 0)
    hipLaunchKernelGGL((k_quant1x16<InT, HAS_RES, SR, GLOBAL, 0, true>), grid, block, 0, st,
                       x, res, ga, key, nblk, packed, scales, out);
  else if (out_kind == 1 && codes)
    hipLaunchKernelGGL((k_quant1x16<InT, HAS_RES, SR, GLOBAL, 1, true>), grid, block, 0, st,
                       x, res, ga, key, nblk, packed, scales, out);
  else if (out_kind == 1)
    hipLaunchKernelGGL((k_quant1x16<InT, HAS_RES, SR, GLOBAL, 1, false>), grid, block, 0, st,
                       x, res, ga, key, nblk, packed, scales, out);
  else if (codes)
    hipLaunchKernelGGL((k_quant1x16<InT, HAS_RES, SR, GLOBAL, 2, true>), grid, block, 0, st,
                       x, res, ga, key, nblk, packed, scales, out);
  else
    hipLaunchKernelGGL((k_quant1x16<InT, HAS_RES, SR, GLOBAL, 2, false>), grid, block, 0, st,
                       x, res, ga, key, nblk, packed, scales, out);
  return (int)hipGetLastError();
}

template <typename InT, bool HAS_RES, bool SR>
static int dispatch_global(const InT* x, float* res, const float* ga, uint32_t key,
                           int64_t nblk, uint8_t* packed, uint8_t* scales, void* out,
                           int out_kind, hipStream_t st) {
  if (ga) return dispatch_out<InT, HAS_RES, SR, true>(x, res, ga, key, nblk, packed, scales, out, out_kind, st);
  return dispatch_out<InT, HAS_RES, SR, false>(x, res, ga, key, nblk, packed, scales, out, out_kind, st);
}

template <typename InT>
static int dispatch_in(const InT* x, float* res, const float* ga, int sr, uint32_t key,
                       int64_t nblk, uint8_t* packed, uint8_t* scales, void* out, int out_kind,
                       hipStream_t st) {
  if (res && sr) return dispatch_global<InT, true, true>(x, res, ga, key, nblk, packed, scales, out, out_kind, st);
  if (res) return dispatch_global<InT, true, false>(x, res, ga, key, nblk, packed, scales, out, out_kind, st);
  if (sr) return dispatch_global<InT, false, true>(x, res, ga, key, nblk, packed, scales, out, out_kind, st);
  return dispatch_global<InT, false, false>(x, res, ga, key, nblk, packed, scales, out, out_kind, st);
}

int launch_quant1x16(const void* x, int in_bf16, int64_t M, int64_t K, float* residual,
                     const float* global_amax, int sr, uint32_t seed, uint32_t step,
                     uint8_t* packed, uint8_t* scales, void* out, int out_kind, void* stream) {
  const int64_t nblk = M * K / 16;
  if (nblk == 0) return 0;
  const uint32_t key = rng_key_host(seed, step);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (in_bf16)
    return dispatch_in(reinterpret_cast<const uint16_t*>(x), residual, global_amax, sr, key, nblk,
                       packed, scales, out, out_kind, st);
  return dispatch_in(reinterpret_cast<const float*>(x), residual, global_amax, sr, key, nblk,
                     packed, scales, out, out_kind, st);
}

// ------------------------------------------------------------- dequantize

// fp4-train, API: dequantize(packed, scale, M, K) -> bf16.  One lane per
// 16-element block: x_hat = (val * s) * S_dec.
template <int SMODE, bool TILE16, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ global_amax,
                                                      float D, int64_t nbk, int64_t nblk,
                                                      void* __restrict__ out) {
  const int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= nblk) return;
  int64_t m = 0, b = blk;
  if (SMODE == 2 || TILE16) { m = blk / nbk; b = blk - m * nbk; }
  const int64_t sidx = TILE16 ? (m >> 4) * nbk + b : blk;
  const float s = e4m3_decode(scales[sidx]);
  float S_dec = 1.0f;
  if (SMODE == 1) S_dec = global_amax[0] / D;
  if (SMODE == 2) S_dec = global_amax[m] / D;
  const uint2 c = reinterpret_cast<const uint2*>(packed)[blk];
  float xh[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t code = ((i < 8 ? c.x : c.y) >> (4 * (i & 7))) & 0xFu;
    const uint32_t mag = code & 7u;
    const float q = mag <= 4u ? (float)mag * 0.5f : (mag == 5u ? 3.0f : (mag == 6u ? 4.0f : 6.0f));
    const float val = (code & 8u) ? -q : q;
    xh[i] = (val * s) * S_dec;
  }
  if (BF16OUT) store16_bf16(reinterpret_cast<uint16_t*>(out) + blk * 16, xh);
  else store16(reinterpret_cast<float*>(out) + blk * 16, xh);
}

template <int SMODE, bool TILE16>
static int dq_out(const uint8_t* p, const uint8_t* s, const float* ga, float D, int64_t nbk,
                  int64_t nblk, void* out, int out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)((nblk + kThreads - 1) / kThreads)), block(kThreads);
  if (out_bf16)
    hipLaunchKernelGGL((k_dequant<SMODE, TILE16, true>), grid, block, 0, st, p, s, ga, D, nbk, nblk, out);
  else
    hipLaunchKernelGGL((k_dequant<SMODE, TILE16, false>), grid, block, 0, st, p, s, ga, D, nbk, nblk, out);
  return (int)hipGetLastError();
}

int launch_dequant(const uint8_t* packed, const uint8_t* scales, int64_t M, int64_t K,
                   int tile16, const float* global_amax, int scale_mode, float bound,
                   void* out, int out_bf16, void* stream) {
  const int64_t nbk = K / 16, nblk = M * nbk;
  if (nblk == 0) return 0;
  const float D = 6.0f * bound;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (tile16) {
    if (scale_mode == 1) return dq_out<1, true>(packed, scales, global_amax, D, nbk, nblk, out, out_bf16, st);
    return dq_out<0, true>(packed, scales, global_amax, D, nbk, nblk, out, out_bf16, st);
  }
  if (scale_mode == 1) return dq_out<1, false>(packed, scales, global_amax, D, nbk, nblk, out, out_bf16, st);
  if (scale_mode == 2) return dq_out<2, false>(packed, scales, global_amax, D, nbk, nblk, out, out_bf16, st);
  return dq_out<0, false>(packed, scales, global_amax, D, nbk, nblk, out, out_bf16, st);
}

}  // namespace nvfp4
