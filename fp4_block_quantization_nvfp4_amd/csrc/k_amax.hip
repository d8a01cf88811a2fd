// Global amax A = NaN-dropping max of |x'| (x' = x + residual), per tensor
// or per row.  Four-over-six pull request, What: a scalar global_amax selects
// per-tensor scaling and a (rows,) vector the row-wise variant; CuTe DSL
// kernel Design: NaN-dropping max (an all-NaN set gives 0).
//
// Per tensor: two passes.  Pass 1 streams the tensor with 128-bit loads in a
// grid-stride loop (without a residual: flat 16-byte chunks, four in flight
// per lane, nontemporal; with one: 16 elements of x and of the residual per
// lane and step), reduces inside the wave with cross-lane max, then across
// the workgroup in LDS, and writes one partial per workgroup into the
// caller's workspace.  Pass 2 (one workgroup)
// reduces the partials and writes A.  Max is exact and order-free, so the
// result does not depend on the launch geometry.  Per row: one workgroup per
// row, same reductions.
#include <mutex>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"
#include "nvfp4_plan.hpp"

namespace nvfp4 {


NV_DEV float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Workgroup max of one value per lane; every lane gets the result.
NV_DEV float block_max(float v, float* lds) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int i = 0; i < nw; ++i) r = fmaxf(r, lds[i]);
  return r;
}

template <typename InT, bool HAS_RES>
NV_DEV float group_absmax(const InT* x, const float* res, int64_t g) {
  float xv[16];
  load16(x + g * 16, xv);
  if (HAS_RES) {
    float r[16];
    load16(res + g * 16, r);
#pragma unroll
    for (int i = 0; i < 16; ++i) xv[i] = xv[i] + r[i];
  }
  // magnitudes compare as integers; a NaN (above 0x7F800000) sends the
  // group to the NaN-dropping form
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t b = f2bits(xv[i]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  if (m <= 0x7F800000u) return bits2f(m);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, abs_nan0(xv[i]));
  return a;
}

template <typename InT, bool HAS_RES>
__global__ __launch_bounds__(kAmaxThreads) void k_amax_partial(const InT* __restrict__ x,
                                                               const float* __restrict__ res,
                                                               int64_t ngroups,
                                                               float* __restrict__ partial) {
  __shared__ float lds[kAmaxThreads / 64];
  float a = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  for (int64_t g = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; g < ngroups; g += stride)
    a = fmaxf(a, group_absmax<InT, HAS_RES>(x, res, g));
  a = block_max(a, lds);
  if (threadIdx.x == 0) partial[blockIdx.x] = a;
}

// Pass 1 without a residual: the tensor as a flat run of 16-byte chunks
// (8 bf16 or 4 fp32 values), consecutive lanes on consecutive chunks (each
// load instruction of a workgroup reads 4 KB contiguous) and kAmaxUnroll
// chunks in flight per lane, read with nontemporal loads (the tensor is not
// reused from the caches; a plain read stream measured about 13% slower).
// Magnitude bit patterns are maxed as integers (bf16: both halves of a word
// at once); a lane whose maximum pattern is a NaN scans its chunks again
// dropping NaNs.
constexpr int kAmaxUnroll = 4;
typedef unsigned int nv_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short nv_u16x2 __attribute__((ext_vector_type(2)));

NV_DEV uint4 ld_nt(const uint4* p) {
  const nv_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nv_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// running max of magnitude patterns: bf16 keeps two 16-bit lanes in a word
NV_DEV uint32_t chunk_max(uint32_t m, const uint4 v, const uint16_t*) {
  const uint32_t w[4] = {v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu};
  nv_u16x2 a = __builtin_bit_cast(nv_u16x2, m);
#pragma unroll
  for (int i = 0; i < 4; ++i) a = __builtin_elementwise_max(a, __builtin_bit_cast(nv_u16x2, w[i]));
  return __builtin_bit_cast(uint32_t, a);
}
NV_DEV uint32_t chunk_max(uint32_t m, const uint4 v, const float*) {
  const uint32_t w[4] = {v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu, v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu};
#pragma unroll
  for (int i = 0; i < 4; ++i) m = w[i] > m ? w[i] : m;
  return m;
}
// the running max as an fp32 pattern, and whether it is a NaN
NV_DEV uint32_t max_bits(uint32_t m, const uint16_t*) {
  const uint32_t h = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
  return h << 16;
}
NV_DEV uint32_t max_bits(uint32_t m, const float*) { return m; }
// NaN-dropping max of one chunk's magnitudes as an fp32 pattern
NV_DEV uint32_t chunk_max_nan_drop(const uint4 v, const uint16_t*) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = ((w[i >> 1] >> (16 * (i & 1))) & 0x7FFFu) << 16;
    if (h <= 0x7F800000u && h > m) m = h;
  }
  return m;
}
NV_DEV uint32_t chunk_max_nan_drop(const uint4 v, const float*) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = w[i] & 0x7FFFFFFFu;
    if (b <= 0x7F800000u && b > m) m = b;
  }
  return m;
}

template <typename InT>
__global__ __launch_bounds__(kAmaxThreads) void k_amax_stream(const uint4* __restrict__ x, int64_t n16,
                                                              float* __restrict__ partial) {
  __shared__ float lds[kAmaxThreads / 64];
  const int64_t first = (int64_t)blockIdx.x * (kAmaxThreads * kAmaxUnroll) + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * (kAmaxThreads * kAmaxUnroll);
  uint32_t m = 0;
  for (int64_t i = first; i < n16; i += stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kAmaxThreads;
      v[u] = j < n16 ? ld_nt(x + j) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = chunk_max(m, v[u], static_cast<const InT*>(nullptr));
  }
  uint32_t mb = max_bits(m, static_cast<const InT*>(nullptr));
  if (mb > 0x7F800000u) {  // a NaN among this lane's chunks: scan them again, dropping NaNs
    mb = 0;
    for (int64_t i = first; i < n16; i += stride)
      for (int u = 0; u < kAmaxUnroll; ++u) {
        const int64_t j = i + (int64_t)u * kAmaxThreads;
        if (j < n16) {
          const uint32_t c = chunk_max_nan_drop(x[j], static_cast<const InT*>(nullptr));
          mb = c > mb ? c : mb;
        }
      }
  }
  const float a = block_max(bits2f(mb), lds);
  if (threadIdx.x == 0) partial[blockIdx.x] = a;
}

__global__ __launch_bounds__(kAmaxThreads) void k_amax_final(const float* __restrict__ partial,
                                                             int n, float* __restrict__ out) {
  __shared__ float lds[kAmaxThreads / 64];
  float a = 0.0f;
  for (int i = threadIdx.x; i < n; i += kAmaxThreads) a = fmaxf(a, partial[i]);
  a = block_max(a, lds);
  if (threadIdx.x == 0) out[0] = a;
}

template <typename InT, bool HAS_RES>
__global__ __launch_bounds__(kAmaxThreads) void k_amax_rows(const InT* __restrict__ x,
                                                            const float* __restrict__ res,
                                                            int64_t M, int64_t K,
                                                            float* __restrict__ out) {
  __shared__ float lds[kAmaxThreads / 64];
  const int64_t nbk = K / 16;
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    float a = 0.0f;
    for (int64_t b = threadIdx.x; b < nbk; b += kAmaxThreads)
      a = fmaxf(a, group_absmax<InT, HAS_RES>(x + m * K, HAS_RES ? res + m * K : res, b));
    a = block_max(a, lds);
    if (threadIdx.x == 0) out[m] = a;
  }
}

size_t amax_workspace_bytes(int64_t M, int64_t K) {
  return (size_t)amax_partial_groups(M, K) * sizeof(float);
}

template <typename InT>
static int amax_typed(const InT* x, int64_t M, int64_t K, const float* res, int mode,
                      float* out, float* ws, hipStream_t st) {
  const int64_t ng = M * K / 16;
  if (mode == 2) {
    if (M == 0) return 0;
    const unsigned grid = (unsigned)plan_amax(M, K, 1).grid;
    if (res) hipLaunchKernelGGL((k_amax_rows<InT, true>), dim3(grid), dim3(kAmaxThreads), 0, st, x, res, M, K, out);
    else hipLaunchKernelGGL((k_amax_rows<InT, false>), dim3(grid), dim3(kAmaxThreads), 0, st, x, res, M, K, out);
    return (int)hipGetLastError();
  }
  const int64_t groups = plan_amax(M, K, 0).grid;
  if (ng > 0) {
    if (res)
      hipLaunchKernelGGL((k_amax_partial<InT, true>), dim3((unsigned)groups), dim3(kAmaxThreads), 0, st, x, res, ng, ws);
    else
      hipLaunchKernelGGL((k_amax_stream<InT>), dim3((unsigned)groups), dim3(kAmaxThreads), 0, st,
                         reinterpret_cast<const uint4*>(x), ng * (int64_t)sizeof(InT), ws);
  }
  hipLaunchKernelGGL(k_amax_final, dim3(1), dim3(kAmaxThreads), 0, st, ws, ng > 0 ? (int)groups : 0, out);
  return (int)hipGetLastError();
}

int launch_amax(const void* x, int in_bf16, int64_t M, int64_t K, const float* residual,
                int mode, float* amax_out, void* workspace, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* ws = reinterpret_cast<float*>(workspace);
  if (in_bf16)
    return amax_typed(reinterpret_cast<const uint16_t*>(x), M, K, residual, mode, amax_out, ws, st);
  return amax_typed(reinterpret_cast<const float*>(x), M, K, residual, mode, amax_out, ws, st);
}

// ------------------------------------------------ allocation-free variant
// The per-tensor pass keeps its per-workgroup partial maxima in this
// file-scope device array instead of a caller's workspace.  Every GPU the
// library runs on holds its own copy (kAmaxMaxGroups floats, 8 KiB) until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it only names a stand-in): the device address of the current
// GPU's copy is looked up once per device with hipGetSymbolAddress and kept.
// Nothing needs clearing between calls: pass 1 writes every partial that
// pass 2 reads.  Calls that overlap on one GPU share the array and race.
constexpr int kScratchFloats = kAmaxMaxGroups;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) float scratch[kScratchFloats];

// Device address of the current GPU's scratch array (nullptr and a HIP
// error code on failure).
static float* scratch_for_current_device(int* err) {
  static std::mutex mu;
  static float* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
      return nullptr;
    }
    ptrs[dev] = static_cast<float*>(p);
  }
  return ptrs[dev];
}

int64_t amax_noalloc_max_partials() { return kScratchFloats; }

int launch_amax_noalloc(const void* x, int in_bf16, int64_t M, int64_t K, const float* residual,
                        int mode, float* amax_out, void* stream) {
  if (mode == 2) return launch_amax(x, in_bf16, M, K, residual, mode, amax_out, nullptr, stream);
  if (amax_partial_groups(M, K) > kScratchFloats) return (int)hipErrorInvalidValue;
  int err = 0;
  float* ws = scratch_for_current_device(&err);
  if (!ws) return err;
  return launch_amax(x, in_bf16, M, K, residual, mode, amax_out, ws, stream);
}

}  // namespace nvfp4
