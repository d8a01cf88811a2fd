// Transposition-invariant 2D NVFP4 quantize: one e4m3 scale per 16x16 tile,
// shared by X and X^T, with round-to-nearest or stochastic rounding ("Stable
// FP4 Training via Transposition-Invariant Block Quantization", abstract).
// Rowwise codes [M, K/2] and the same codes transposed [K, M/2] are written in
// one pass (the fused row + column kernel the four-over-six pull request lists
// as a follow-up), so no caller-side transpose is needed.
//
// Mapping: a workgroup of 256 lanes covers a 16-row x 256-column strip, i.e.
// 16 tiles side by side, four per wave.  Lane (t, r) = (tid / 16, tid % 16)
// holds row r of tile t: 16 consecutive elements read with 128-bit loads, so
// each wave reads 16 rows x 128 contiguous bytes.  The tile amax is reduced
// across the 16 lanes of the tile with cross-lane max (all 16 lanes of a tile
// sit in one 16-lane row of the wave).  The rowwise codes go out as one 8-byte
// store per lane.  For the columnwise codes each lane stages its 16 codes as
// bytes in LDS; lane (t, c) then gathers column c of its tile and stores the
// 16 codes of that column (8 bytes) into row k of packed_col.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

constexpr int k2dThreads = 256;

template <typename InT, bool SR, bool GLOBAL, bool COL>
__global__ __launch_bounds__(k2dThreads) void k_quant2d(
    const InT* __restrict__ x, const float* __restrict__ global_amax, uint32_t key, int64_t M,
    int64_t K, uint8_t* __restrict__ packed_row, uint8_t* __restrict__ packed_col,
    uint8_t* __restrict__ tile_scales, int64_t ncolg) {
  __shared__ uint4 stage[k2dThreads];
  const int t = threadIdx.x >> 4, r = threadIdx.x & 15;
  const int64_t strip = (int64_t)blockIdx.x / ncolg, cg = (int64_t)blockIdx.x - strip * ncolg;
  const int64_t col0 = cg * 256 + 16 * t;
  const int64_t row0 = strip * 16;
  const int64_t row = row0 + r;
  const bool active = col0 < K;  // uniform over the 16 lanes of a tile

  float S_dec = 1.0f, mul = 0.0f;
  if (GLOBAL) {
    float S_enc;
    global_scales(global_amax[0], 2688.0f, S_enc, S_dec);
    mul = S_enc * (1.0f / 6.0f);
  }

  float xv[16];
  float a = 0.0f;
  if (active) {
    load16(x + row * K + col0, xv);
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xv[i]));
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));

  uint32_t codes[16];
  if (active) {
    float sigma = GLOBAL ? a * mul : a / 6.0f;
    sigma = fminf(sigma, kE4m3Max);
    const uint32_t sc = e4m3_encode(sigma);
    const float s = e4m3_decode(sc);
    const float rho = encode_reciprocal(s, S_dec);
    uint32_t w[8];
    if (SR) {
      const uint32_t p0 = (uint32_t)((row * K + col0) >> 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = pcg_hash((p0 + j) ^ key);
    }
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = fabsf(xv[i]) * rho;
      float q;
      uint32_t mag;
      if (SR) mag = e2m1_sr(v, (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu, q);
      else mag = e2m1_rtn(v, q);
      const uint32_t neg = (v != v) ? 0u : (f2bits(xv[i]) >> 31);
      codes[i] = mag | (neg << 3);
      if (i < 8) c0 |= codes[i] << (4 * i);
      else c1 |= codes[i] << (4 * (i - 8));
    }
    *reinterpret_cast<uint2*>(packed_row + row * (K / 2) + col0 / 2) = make_uint2(c0, c1);
    if (r == 0) tile_scales[(row0 / 16) * (K / 16) + col0 / 16] = (uint8_t)sc;
  }
  if (COL) {
    if (active) {
      uint32_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = codes[4 * j] | (codes[4 * j + 1] << 8) | (codes[4 * j + 2] << 16) | (codes[4 * j + 3] << 24);
      stage[threadIdx.x] = make_uint4(b[0], b[1], b[2], b[3]);
    }
    __syncthreads();
    if (active) {
      const uint8_t* tile = reinterpret_cast<const uint8_t*>(&stage[16 * t]);
      const int c = r;  // this lane now handles column c of its tile
      uint32_t o0 = 0, o1 = 0;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const uint32_t code = tile[16 * rr + c];
        if (rr < 8) o0 |= code << (4 * rr);
        else o1 |= code << (4 * (rr - 8));
      }
      *reinterpret_cast<uint2*>(packed_col + (col0 + c) * (M / 2) + row0 / 2) = make_uint2(o0, o1);
    }
  }
}

template <typename InT, bool SR, bool GLOBAL>
static int launch2d_col(const InT* x, const float* ga, uint32_t key, int64_t M, int64_t K,
                        uint8_t* pr, uint8_t* pc, uint8_t* ts, hipStream_t st) {
  const int64_t ncolg = (K + 255) / 256;
  const dim3 grid((unsigned)(ncolg * (M / 16))), block(k2dThreads);
  if (pc) hipLaunchKernelGGL((k_quant2d<InT, SR, GLOBAL, true>), grid, block, 0, st, x, ga, key, M, K, pr, pc, ts, ncolg);
  else hipLaunchKernelGGL((k_quant2d<InT, SR, GLOBAL, false>), grid, block, 0, st, x, ga, key, M, K, pr, pc, ts, ncolg);
  return (int)hipGetLastError();
}

template <typename InT>
static int launch2d_typed(const InT* x, const float* ga, int sr, uint32_t key, int64_t M,
                          int64_t K, uint8_t* pr, uint8_t* pc, uint8_t* ts, hipStream_t st) {
  if (sr && ga) return launch2d_col<InT, true, true>(x, ga, key, M, K, pr, pc, ts, st);
  if (sr) return launch2d_col<InT, true, false>(x, ga, key, M, K, pr, pc, ts, st);
  if (ga) return launch2d_col<InT, false, true>(x, ga, key, M, K, pr, pc, ts, st);
  return launch2d_col<InT, false, false>(x, ga, key, M, K, pr, pc, ts, st);
}

int launch_quant2d(const void* x, int in_bf16, int64_t M, int64_t K, const float* global_amax,
                   int sr, uint32_t seed, uint32_t step, uint8_t* packed_row,
                   uint8_t* packed_col, uint8_t* tile_scales, void* stream) {
  if (M == 0 || K == 0) return 0;
  const uint32_t key = rng_key_host(seed, step);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (in_bf16)
    return launch2d_typed(reinterpret_cast<const uint16_t*>(x), global_amax, sr, key, M, K,
                          packed_row, packed_col, tile_scales, st);
  return launch2d_typed(reinterpret_cast<const float*>(x), global_amax, sr, key, M, K, packed_row,
                        packed_col, tile_scales, st);
}

}  // namespace nvfp4
