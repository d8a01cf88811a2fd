// Four-over-six NVFP4 quantize on 1x16 blocks (four-over-six pull request
// "Add NVFP4 four-over-six (row-wise) quantization to the training
// prototype": What, the two numeric details, CuTe DSL kernel Design).
//
// Every block is encoded twice with round-to-nearest: map-to-6 with
// sigma6 = (block_amax / 6) * S_enc and map-to-4 with sigma4 = sigma6 * 1.5
// (each capped at 448 by a NaN-dropping min before its e4m3 cast).  For
// each candidate the dequantization error of every element is taken against
// d = ((val * s) * A) / (6 * bound) with a true division, as |x - d| (MAE) or
// (x - d)^2 (MSE), and summed strictly in element order 0..15.  The
// candidate with the strictly lower sum is stored; ties and NaN keep
// map-to-6.
//
// Mapping: one workgroup per row (grid-stride over rows), one lane per
// 16-element block of the row.  The per-row global amax is either read or
// reduced by the workgroup in the same kernel (a first sweep over the row,
// then the encode sweep re-reads the row, which is still in L2).  The work
// is HBM streaming plus per-element VALU arithmetic; no LDS beyond the
// workgroup reduction and no MFMA.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

constexpr int k46MaxThreads = 1024;

NV_DEV float wave_max46(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <typename InT>
NV_DEV float block_absmax16(const InT* p, float xv[16]) {
  load16(p, xv);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xv[i]));
  return a;
}

// One candidate: codes (two u32 of packed nibbles) and the error sum.
template <bool MSE>
NV_DEV float candidate(const float xv[16], float s, float rho, float A, float D, uint32_t& c0,
                       uint32_t& c1) {
  float E = 0.0f;
  c0 = 0;
  c1 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float ax = fabsf(xv[i]);
    const float v = ax * rho;
    float q;
    const uint32_t mag = e2m1_rtn(v, q);
    const uint32_t neg = (v != v) ? 0u : (f2bits(xv[i]) >> 31);
    const uint32_t code = mag | (neg << 3);
    if (i < 8) c0 |= code << (4 * i);
    else c1 |= code << (4 * (i - 8));
    // |x - d| and (x - d)^2 are unchanged when both signs are flipped, so
    // the error is taken on magnitudes.
    const float d = ((q * s) * A) / D;
    const float t = ax - d;
    const float e = MSE ? t * t : fabsf(t);
    E = (i == 0) ? e : E + e;
  }
  return E;
}

template <typename InT, bool MSE, int MODE>
__global__ __launch_bounds__(k46MaxThreads) void k_4over6(const InT* __restrict__ x,
                                                          float* __restrict__ amax, float D,
                                                          int64_t M, int64_t K,
                                                          uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ scales) {
  // MODE 1: one amax for the tensor; 2: row amax given; 3: row amax computed here.
  __shared__ float lds[k46MaxThreads / 64];
  const int64_t nbk = K / 16;
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    const InT* xr = x + m * K;
    float A;
    if (MODE == 1) A = amax[0];
    else if (MODE == 2) A = amax[m];
    else {
      float a = 0.0f, xv[16];
      for (int64_t b = threadIdx.x; b < nbk; b += blockDim.x) a = fmaxf(a, block_absmax16(xr + b * 16, xv));
      a = wave_max46(a);
      __syncthreads();
      if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = a;
      __syncthreads();
      A = 0.0f;
      for (int i = 0; i < (int)(blockDim.x >> 6); ++i) A = fmaxf(A, lds[i]);
      if (threadIdx.x == 0) amax[m] = A;
    }
    float S_enc, S_dec;
    global_scales(A, D, S_enc, S_dec);
    for (int64_t b = threadIdx.x; b < nbk; b += blockDim.x) {
      float xv[16];
      const float a = block_absmax16(xr + b * 16, xv);
      const float sig6r = (a / 6.0f) * S_enc;
      const float sig4r = sig6r * 1.5f;
      const uint32_t k6 = e4m3_encode(fminf(sig6r, kE4m3Max));
      const uint32_t k4 = e4m3_encode(fminf(sig4r, kE4m3Max));
      const float s6 = e4m3_decode(k6), s4 = e4m3_decode(k4);
      uint32_t a0, a1, b0, b1;
      const float E6 = candidate<MSE>(xv, s6, encode_reciprocal(s6, S_dec), A, D, a0, a1);
      const float E4 = candidate<MSE>(xv, s4, encode_reciprocal(s4, S_dec), A, D, b0, b1);
      const bool pick4 = E4 < E6;
      const int64_t blk = m * nbk + b;
      reinterpret_cast<uint2*>(packed)[blk] = pick4 ? make_uint2(b0, b1) : make_uint2(a0, a1);
      scales[blk] = (uint8_t)(pick4 ? k4 : k6);
    }
  }
}

template <typename InT, bool MSE>
static int launch46_mode(const InT* x, float* amax, int mode, int amax_is_input, float D,
                         int64_t M, int64_t K, uint8_t* packed, uint8_t* scales, hipStream_t st) {
  const int64_t nbk = K / 16;
  int threads = (int)((nbk + 63) / 64 * 64);
  if (threads > k46MaxThreads) threads = k46MaxThreads;
  if (threads < 64) threads = 64;
  const unsigned grid = (unsigned)(M < 1048576 ? M : 1048576);
  if (mode == 1)
    hipLaunchKernelGGL((k_4over6<InT, MSE, 1>), dim3(grid), dim3(threads), 0, st, x, amax, D, M, K, packed, scales);
  else if (amax_is_input)
    hipLaunchKernelGGL((k_4over6<InT, MSE, 2>), dim3(grid), dim3(threads), 0, st, x, amax, D, M, K, packed, scales);
  else
    hipLaunchKernelGGL((k_4over6<InT, MSE, 3>), dim3(grid), dim3(threads), 0, st, x, amax, D, M, K, packed, scales);
  return (int)hipGetLastError();
}

int launch_4over6(const void* x, int in_bf16, int64_t M, int64_t K, float* amax, int mode,
                  int amax_is_input, int mse, float bound, uint8_t* packed, uint8_t* scales,
                  void* stream) {
  if (M == 0 || K == 0) return 0;
  const float D = 6.0f * bound;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (in_bf16) {
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    return mse ? launch46_mode<uint16_t, true>(xb, amax, mode, amax_is_input, D, M, K, packed, scales, st)
               : launch46_mode<uint16_t, false>(xb, amax, mode, amax_is_input, D, M, K, packed, scales, st);
  }
  const float* xf = reinterpret_cast<const float*>(x);
  return mse ? launch46_mode<float, true>(xf, amax, mode, amax_is_input, D, M, K, packed, scales, st)
             : launch46_mode<float, false>(xf, amax, mode, amax_is_input, D, M, K, packed, scales, st);
}

}  // namespace nvfp4
