// Global amax A = NaN-dropping max of |x'| (x' = x + residual), per tensor
// or per row.  Four-over-six pull request, What: a scalar global_amax selects
// per-tensor scaling and a (rows,) vector the row-wise variant; CuTe DSL
// kernel Design: NaN-dropping max (an all-NaN set gives 0).
//
// Per tensor: two passes.  Pass 1 streams the tensor with 128-bit loads in a
// grid-stride loop (each lane 16 elements per step), reduces inside the wave
// with cross-lane max, then across the workgroup in LDS, and writes one
// partial per workgroup into the caller's workspace.  Pass 2 (one workgroup)
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
    if (res) hipLaunchKernelGGL((k_amax_partial<InT, true>), dim3((unsigned)groups), dim3(kAmaxThreads), 0, st, x, res, ng, ws);
    else hipLaunchKernelGGL((k_amax_partial<InT, false>), dim3((unsigned)groups), dim3(kAmaxThreads), 0, st, x, res, ng, ws);
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
