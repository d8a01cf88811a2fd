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
// Generic kernel (fp32 input, or rows longer than 16384): one workgroup per
// row (grid-stride over rows), one lane per 16-element block of the row.  The
// per-row global amax is either read or reduced by the workgroup in the same
// kernel (a first sweep over the row, then the encode sweep re-reads the row,
// which is still in L2).  Each block takes fos_block: hardware encode of both
// candidates, the certified choice, exact sums for undecided blocks and the
// software candidate outside the range guards; the encode reciprocals of all
// scale codes are tabulated in LDS per row.  The work is HBM streaming plus
// per-element VALU arithmetic; no MFMA.
#include "nvfp4_device.hpp"
#include "nvfp4_fos.hpp"
#include "nvfp4_launch.hpp"
#include "nvfp4_plan.hpp"

namespace nvfp4 {

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
  for (int i = 0; i < 16; ++i) a = fmaxf(a, abs_nan0(xv[i]));
  return a;
}

template <typename InT, bool MSE, int MODE>
__global__ __launch_bounds__(k46MaxThreads) void k_4over6(const InT* __restrict__ x,
                                                          float* __restrict__ amax, float D,
                                                          int64_t M, int64_t K,
                                                          uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ scales) {
  // MODE 1: one amax for the tensor; 2: row amax given; 3: row amax computed here.
  __shared__ float lds[k46MaxThreads / 64];
  __shared__ float rhoT[128];
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
      if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = a;
      __syncthreads();
      A = 0.0f;
      for (int i = 0; i < (int)(blockDim.x >> 6); ++i) A = fmaxf(A, lds[i]);
      if (threadIdx.x == 0) amax[m] = A;
    }
    float S_enc, S_dec;
    global_scales(A, D, S_enc, S_dec);
    for (int k = threadIdx.x; k < 127; k += blockDim.x) rhoT[k] = encode_reciprocal(e4m3_decode(k), S_dec);
    __syncthreads();
    const bool lean = fos_row_in_range(A, S_dec);
    for (int64_t b = threadIdx.x; b < nbk; b += blockDim.x) {
      float xv[16];
      load16(xr + b * 16, xv);
      uint32_t c[2];
      const uint32_t sbyte = fos_block_f32<MSE, MODE != 3>(xv, lean, S_enc, S_dec, A, D, rhoT, c);
      const int64_t blk = m * nbk + b;
      st_nt_u2(reinterpret_cast<uint2*>(packed) + blk, c[0], c[1]);
      st_nt_u8(scales + blk, sbyte);
    }
    __syncthreads();  // lds and rhoT are rewritten for the next row
  }
}

// ---------------------------------------------------------------------------
// Row-per-workgroup kernel for bf16 input (K <= 16384).  Same numerics as
// above, with exact rewrites of the per-element work:
//  * e2m1 encode by the gfx950 packed fp32 -> fp4 conversion (scale 1.0),
//    which rounds to nearest-even and saturates at +-6 exactly like the
//    software encoder for every finite and infinite input (an exhaustive
//    scan of all fp32 patterns); the block scale bytes come from the hardware
//    fp32 -> e4m3 conversion, equal to the software encoder on [0, 448].
//  * The candidate choice is certified from error sums in the scaled
//    domain (fos_block); only undecided blocks compute the per-element
//    dequant values with true divisions.
//  * The encode reciprocals of all 127 scale codes, and the products
//    W = s * S_dec of the error bound, are tabulated in LDS once per row
//    (one correctly rounded reciprocal per lane).
//  * a / 6 uses reciprocal-multiply plus one exact FMA remainder correction
//    where that is proven correctly rounded, else the true division.
// A two-wave workgroup owns one row: it loads the row (R blocks per lane)
// into registers, reduces the row amax (when it is computed here), builds
// the reciprocal table, then encodes its blocks.

typedef unsigned short nv_us2 __attribute__((ext_vector_type(2)));

// Max of the 16 bf16 magnitudes of a block as 16-bit patterns (for
// non-NaN values the integer order is the value order; a NaN compares above
// every finite value and infinity).
NV_DEV uint32_t absmax_bits(const uint4 r0, const uint4 r1) {
  const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  nv_us2 m = __builtin_bit_cast(nv_us2, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(nv_us2, w[i] & 0x7FFF7FFFu));
  return m.x > m.y ? m.x : m.y;
}

// NaN-dropping variant (the block holds a NaN): max over non-NaN magnitudes.
NV_DEV uint32_t absmax_bits_nan_drop(const uint4 r0, const uint4 r1) {
  const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0x7FFFu;
    if (h <= 0x7F80u && h > m) m = h;
  }
  return m;
}

NV_DEV void unpack16(const uint4 r0, const uint4 r1, float xv[16]) {
  const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xv[2 * i] = bits2f(w[i] << 16);
    xv[2 * i + 1] = bits2f(w[i] & 0xFFFF0000u);
  }
}

// Lane-wise max of two packed pairs of u16.
NV_DEV uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(nv_us2, a),
                                                                 __builtin_bit_cast(nv_us2, b)));
}

// Wave-wide max of two packed u16 values, returned to every lane (uniform):
// quad permutations, half-row and row mirrors (DPP, no LDS), then the four
// 16-lane rows are combined through lane reads.
NV_DEV uint32_t wave_max_pk_u16(uint32_t v) {
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row half mirror
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return pk_max_u16(pk_max_u16(r0, r1), pk_max_u16(r2, r3));
}

// One workgroup of kRowThreads lanes (two waves) per row; lane t owns blocks
// t, t + kRowThreads, ... (R per lane).

template <bool MSE, int MODE, int R>
__global__ __launch_bounds__(kRowThreads) void k_4over6_rows(const uint16_t* __restrict__ x,
                                                             float* __restrict__ amax, float D,
                                                             int64_t M, int64_t K,
                                                             uint8_t* __restrict__ packed,
                                                             uint8_t* __restrict__ scales) {
  __shared__ float rhoT[128];
  __shared__ float WT[128];
  __shared__ uint32_t red[kRowThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nbk = (int)(K >> 4);
  const uint16_t* xr = x + row * K;

  // A lane past the row's last block loads the last block again (no branch,
  // no register clear): its amax cannot exceed the row's and it encodes
  // nothing.
  uint4 raw[R][2];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int b = tid + kRowThreads * j;
    const uint32_t off = (uint32_t)(b < nbk ? b : nbk - 1) * 32u;  // bytes; nbk <= 1024 here
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(xr) + off);
    raw[j][0] = p[0];
    raw[j][1] = p[1];
  }
  // NaN-dropping block amaxes as bf16 bit patterns; bit j of nan_blocks marks
  // a block that holds a NaN (it never takes the lean path: the hardware
  // encoder gives a negative NaN the code 0xF)
  uint32_t ab[R];
  uint32_t lane_max = 0, nan_blocks = 0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    ab[j] = absmax_bits(raw[j][0], raw[j][1]);
    if (ab[j] > 0x7F80u) {
      nan_blocks |= 1u << j;
      ab[j] = absmax_bits_nan_drop(raw[j][0], raw[j][1]);
    }
    lane_max = ab[j] > lane_max ? ab[j] : lane_max;
  }

  float A;
  if (MODE == 1) {
    A = amax[0];
  } else if (MODE == 2) {
    A = amax[row];
  } else {
    const uint32_t wm = wave_max_pk_u16(lane_max);
    if (lane == 0) red[wave] = wm;
    __syncthreads();
    const uint32_t m = pk_max_u16(red[0], red[1]);
    A = bits2f((m & 0xFFFFu) << 16);
    if (tid == 0) amax[row] = A;
  }
  float S_enc, S_dec;
  global_scales(A, D, S_enc, S_dec);
  if (tid < 127) {
    const float s = hw_e4m3_value<0>((uint32_t)tid);
    rhoT[tid] = encode_reciprocal(s, S_dec);
    WT[tid] = s * S_dec;
  }
  __syncthreads();

  // in a row (or tensor) in range, plain blocks skip the range guards; with
  // the row's own amax (computed here) every finite block has a <= A
  const bool lean = fos_row_in_range(A, S_dec);
  uint2* prow = reinterpret_cast<uint2*>(packed) + row * nbk;
  uint8_t* srow = scales + row * nbk;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int b = tid + kRowThreads * j;
    if (b >= nbk) continue;
    float xv[16];
    unpack16(raw[j][0], raw[j][1], xv);
    uint32_t c[2];
    // plain: no NaN, finite amax of at least 2^-117 and (row amax given or
    // per tensor) a <= A; with the row's own amax a <= A always holds
    const float a = bits2f(ab[j] << 16);
    const bool plain = lean && !((nan_blocks >> j) & 1u) && ab[j] < 0x7F80u && ab[j] >= 0x0500u &&
                       (MODE == 3 || a <= A);
    const uint32_t sbyte = MODE == 3
        ? fos_block_plain<MSE, false, true>(xv, a, plain, S_enc, S_dec, A, D, rhoT, c, WT)
        : fos_block_plain<MSE, true, true>(xv, a, plain, S_enc, S_dec, A, D, rhoT, c, WT);
    st_nt_u2(prow + b, c[0], c[1]);
    st_nt_u8(srow + b, sbyte);
  }
}

// One launch per chunk of at most kRowChunk rows (grid x workgroup stays far
// below 2^32 work-items); a chunk's pointers start at its first row.
template <bool MSE, int MODE>
static int launch_rows_R(int R, const uint16_t* x, float* amax, float D, int64_t M, int64_t K,
                         uint8_t* packed, uint8_t* scales, hipStream_t st) {
  const LaunchPlan pl = plan_4over6(1, M, K);
  for (int64_t l = 0; l < pl.launches; ++l) {
    const int64_t m0 = l * kRowChunk, rows = (M - m0) < kRowChunk ? (M - m0) : kRowChunk;
    const uint16_t* xc = x + m0 * K;
    float* ac = MODE == 1 ? amax : amax + m0;
    uint8_t* pc = packed + m0 * (K / 2);
    uint8_t* sc = scales + m0 * (K / 16);
    const dim3 grid((unsigned)rows), block(pl.block);
#define NV46_CASE(RR) \
  case RR: hipLaunchKernelGGL((k_4over6_rows<MSE, MODE, RR>), grid, block, 0, st, xc, ac, D, rows, K, pc, sc); break;
    switch (R) {
      NV46_CASE(1) NV46_CASE(2) NV46_CASE(3) NV46_CASE(4) NV46_CASE(5) NV46_CASE(6) NV46_CASE(7) NV46_CASE(8)
      default: return (int)hipErrorInvalidValue;
    }
#undef NV46_CASE
    const int e = (int)hipGetLastError();
    if (e) return e;
  }
  return 0;
}

template <typename InT, bool MSE>
static int launch46_mode(const InT* x, float* amax, int mode, int amax_is_input, float D,
                         int64_t M, int64_t K, uint8_t* packed, uint8_t* scales, hipStream_t st) {
  const LaunchPlan pl = plan_4over6(sizeof(InT) == 2, M, K);
  const int threads = pl.block;
  const unsigned grid = (unsigned)pl.grid;
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
  const int64_t nbk = K / 16;
  if (use_rows_kernel(in_bf16, K)) {
    const int R = (int)((nbk + kRowThreads - 1) / kRowThreads);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    const int md = mode == 1 ? 1 : (amax_is_input ? 2 : 3);
    if (mse) {
      if (md == 1) return launch_rows_R<true, 1>(R, xb, amax, D, M, K, packed, scales, st);
      if (md == 2) return launch_rows_R<true, 2>(R, xb, amax, D, M, K, packed, scales, st);
      return launch_rows_R<true, 3>(R, xb, amax, D, M, K, packed, scales, st);
    }
    if (md == 1) return launch_rows_R<false, 1>(R, xb, amax, D, M, K, packed, scales, st);
    if (md == 2) return launch_rows_R<false, 2>(R, xb, amax, D, M, K, packed, scales, st);
    return launch_rows_R<false, 3>(R, xb, amax, D, M, K, packed, scales, st);
  }
  if (in_bf16) {  // rows longer than the row kernel takes
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    return mse ? launch46_mode<uint16_t, true>(xb, amax, mode, amax_is_input, D, M, K, packed, scales, st)
               : launch46_mode<uint16_t, false>(xb, amax, mode, amax_is_input, D, M, K, packed, scales, st);
  }
  const float* xf = reinterpret_cast<const float*>(x);
  return mse ? launch46_mode<float, true>(xf, amax, mode, amax_is_input, D, M, K, packed, scales, st)
             : launch46_mode<float, false>(xf, amax, mode, amax_is_input, D, M, K, packed, scales, st);
}

}  // namespace nvfp4
