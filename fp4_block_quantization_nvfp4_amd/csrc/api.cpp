// C ABI of libnvfp4: host-side argument validation, then dispatch to the
// kernel launchers.  Validation runs entirely on the host and touches no
// device memory, so every error branch returns before anything is queued.
#include <stdint.h>

#include "../../include/nvfp4.h"
#include "nvfp4_launch.hpp"
#include "nvfp4_plan.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 33;  // pair index (i >> 1) fits 32 bits

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool dtype_ok(int d) { return d == NVFP4_F32 || d == NVFP4_BF16; }

nvfp4_status check_shape(int64_t M, int64_t K, bool tiles) {
  if (M < 0 || K < 0) return NVFP4_E_SHAPE;
  if (K % 16 != 0) return NVFP4_E_SHAPE;
  if (tiles && M % 16 != 0) return NVFP4_E_SHAPE;
  if (K > 0 && M > kMaxElems / K) return NVFP4_E_RANGE;
  return NVFP4_OK;
}

nvfp4_status hip_status(int e) { return e == 0 ? NVFP4_OK : NVFP4_E_HIP; }

}  // namespace

extern "C" {

const char* nvfp4_status_str(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_E_NULL: return "a required pointer is NULL";
    case NVFP4_E_SHAPE: return "bad shape (negative, K % 16 != 0, or M % 16 != 0 for 16x16 tiles)";
    case NVFP4_E_DTYPE: return "unknown dtype";
    case NVFP4_E_ALIGN: return "pointer misaligned";
    case NVFP4_E_ARG: return "bad argument (enum value, bound or workspace size)";
    case NVFP4_E_RANGE: return "tensor too large (M*K > 2^33)";
    case NVFP4_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t nvfp4_amax_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return nvfp4::amax_workspace_bytes(M, K);
}

nvfp4_status nvfp4_amax(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                        const float* residual, nvfp4_scale_mode mode, float* amax_out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (nvfp4_status st = check_shape(M, K, false)) return st;
  if (!dtype_ok(dt)) return NVFP4_E_DTYPE;
  if (mode != NVFP4_SCALE_TENSOR && mode != NVFP4_SCALE_ROW) return NVFP4_E_ARG;
  const bool empty = M == 0 || K == 0;
  if (!amax_out) return NVFP4_E_NULL;
  if (!empty && !x) return NVFP4_E_NULL;
  if (mode == NVFP4_SCALE_TENSOR) {
    if (!workspace) return NVFP4_E_NULL;
    if (workspace_bytes < nvfp4::amax_workspace_bytes(M, K)) return NVFP4_E_ARG;
    if (!aligned(workspace, 4)) return NVFP4_E_ALIGN;
  }
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(amax_out, 4)) return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_amax(x, dt == NVFP4_BF16, M, K, residual,
                                       mode == NVFP4_SCALE_TENSOR ? 1 : 2, amax_out, workspace,
                                       stream));
}

nvfp4_status nvfp4_amax_noalloc(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                const float* residual, nvfp4_scale_mode mode, float* amax_out,
                                void* stream) {
  if (nvfp4_status st = check_shape(M, K, false)) return st;
  if (!dtype_ok(dt)) return NVFP4_E_DTYPE;
  if (mode != NVFP4_SCALE_TENSOR && mode != NVFP4_SCALE_ROW) return NVFP4_E_ARG;
  if (!amax_out) return NVFP4_E_NULL;
  if (M != 0 && K != 0 && !x) return NVFP4_E_NULL;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(amax_out, 4)) return NVFP4_E_ALIGN;
  if (mode == NVFP4_SCALE_TENSOR &&
      nvfp4::amax_partial_groups(M, K) > nvfp4::amax_noalloc_max_partials())
    return NVFP4_E_RANGE;
  return hip_status(nvfp4::launch_amax_noalloc(x, dt == NVFP4_BF16, M, K, residual,
                                               mode == NVFP4_SCALE_TENSOR ? 1 : 2, amax_out, stream));
}

static nvfp4_status quant_common(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                 float* residual, const float* global_amax, nvfp4_round rnd,
                                 uint32_t seed, uint32_t step, uint8_t* packed, uint8_t* scales,
                                 void* out, int out_kind, void* stream) {
  if (nvfp4_status st = check_shape(M, K, false)) return st;
  if (!dtype_ok(dt)) return NVFP4_E_DTYPE;
  if (rnd != NVFP4_RTN && rnd != NVFP4_SR) return NVFP4_E_ARG;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!x) return NVFP4_E_NULL;
  if (out_kind == 0 && (!packed || !scales)) return NVFP4_E_NULL;
  if (out_kind != 0 && !out) return NVFP4_E_NULL;
  if ((packed == nullptr) != (scales == nullptr)) return NVFP4_E_NULL;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(out, 16) || !aligned(packed, 8) ||
      !aligned(global_amax, 4))
    return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_quant1x16(x, dt == NVFP4_BF16, M, K, residual, global_amax,
                                            rnd == NVFP4_SR, seed, step, packed, scales, out,
                                            out_kind, stream));
}

nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                            float* residual, const float* global_amax, nvfp4_round rnd,
                            uint32_t seed, uint32_t step, uint8_t* packed, uint8_t* scales,
                            void* stream) {
  return quant_common(x, dt, M, K, residual, global_amax, rnd, seed, step, packed, scales,
                      nullptr, 0, stream);
}

nvfp4_status nvfp4_qdq(const void* x, nvfp4_dtype dt, int64_t M, int64_t K, float* residual,
                       const float* global_amax, nvfp4_round rnd, uint32_t seed,
                       uint32_t step, void* out, nvfp4_dtype out_dt, uint8_t* packed_opt,
                       uint8_t* scales_opt, void* stream) {
  if (!dtype_ok(out_dt)) return NVFP4_E_DTYPE;
  return quant_common(x, dt, M, K, residual, global_amax, rnd, seed, step, packed_opt,
                      scales_opt, out, out_dt == NVFP4_BF16 ? 1 : 2, stream);
}

nvfp4_status nvfp4_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t M,
                              int64_t K, int tile16, const float* global_amax,
                              nvfp4_scale_mode scale_mode, float bound, void* out,
                              nvfp4_dtype out_dt, void* stream) {
  if (tile16 != 0 && tile16 != 1) return NVFP4_E_ARG;
  if (nvfp4_status st = check_shape(M, K, tile16 == 1)) return st;
  if (!dtype_ok(out_dt)) return NVFP4_E_DTYPE;
  if (scale_mode != NVFP4_SCALE_NONE && scale_mode != NVFP4_SCALE_TENSOR &&
      scale_mode != NVFP4_SCALE_ROW)
    return NVFP4_E_ARG;
  if (tile16 && scale_mode == NVFP4_SCALE_ROW) return NVFP4_E_ARG;
  if (scale_mode != NVFP4_SCALE_NONE && !(bound == 256.0f || bound == 448.0f)) return NVFP4_E_ARG;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!packed || !scales || !out) return NVFP4_E_NULL;
  if (scale_mode != NVFP4_SCALE_NONE && !global_amax) return NVFP4_E_NULL;
  if (!aligned(packed, 8) || !aligned(out, 16) || !aligned(global_amax, 4)) return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_dequant(packed, scales, M, K, tile16,
                                          scale_mode == NVFP4_SCALE_NONE ? nullptr : global_amax,
                                          (int)scale_mode, bound, out, out_dt == NVFP4_BF16,
                                          stream));
}

nvfp4_status nvfp4_quantize_4over6(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                   float* global_amax, nvfp4_scale_mode mode,
                                   int amax_is_input, nvfp4_err err, float bound,
                                   uint8_t* packed, uint8_t* scales, void* stream) {
  if (nvfp4_status st = check_shape(M, K, false)) return st;
  if (!dtype_ok(dt)) return NVFP4_E_DTYPE;
  if (mode != NVFP4_SCALE_TENSOR && mode != NVFP4_SCALE_ROW) return NVFP4_E_ARG;
  if (err != NVFP4_MAE && err != NVFP4_MSE) return NVFP4_E_ARG;
  if (!(bound == 256.0f || bound == 448.0f)) return NVFP4_E_ARG;
  if (mode == NVFP4_SCALE_TENSOR && !amax_is_input) return NVFP4_E_ARG;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!x || !global_amax || !packed || !scales) return NVFP4_E_NULL;
  if (!aligned(x, 16) || !aligned(packed, 8) || !aligned(global_amax, 4)) return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_4over6(x, dt == NVFP4_BF16, M, K, global_amax,
                                         mode == NVFP4_SCALE_TENSOR ? 1 : 2, amax_is_input != 0,
                                         err == NVFP4_MSE, bound, packed, scales, stream));
}

nvfp4_status nvfp4_quantize_2d(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                               const float* global_amax, nvfp4_round rnd, uint32_t seed,
                               uint32_t step, int truncation_free, uint8_t* packed_row,
                               uint8_t* packed_col, uint8_t* tile_scales, void* stream) {
  if (nvfp4_status st = check_shape(M, K, true)) return st;
  if (!dtype_ok(dt)) return NVFP4_E_DTYPE;
  if (rnd != NVFP4_RTN && rnd != NVFP4_SR) return NVFP4_E_ARG;
  if (truncation_free != 0 && truncation_free != 1) return NVFP4_E_ARG;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!x || !packed_row || !tile_scales) return NVFP4_E_NULL;
  if (!aligned(x, 16) || !aligned(packed_row, 8) || !aligned(packed_col, 8) ||
      !aligned(global_amax, 4))
    return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_quant2d(x, dt == NVFP4_BF16, M, K, global_amax,
                                          rnd == NVFP4_SR, seed, step, truncation_free,
                                          packed_row, packed_col, tile_scales, stream));
}

nvfp4_status nvfp4_quantize_rowcol(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                   const float* global_amax, int four_over_six, nvfp4_err err,
                                   float bound, uint8_t* packed_row, uint8_t* scales_row,
                                   uint8_t* packed_col, uint8_t* scales_col, void* stream) {
  if (nvfp4_status st = check_shape(M, K, true)) return st;
  if (!dtype_ok(dt)) return NVFP4_E_DTYPE;
  if (four_over_six != 0 && four_over_six != 1) return NVFP4_E_ARG;
  if (err != NVFP4_MAE && err != NVFP4_MSE) return NVFP4_E_ARG;
  if (four_over_six ? !(bound == 256.0f || bound == 448.0f) : bound != 448.0f) return NVFP4_E_ARG;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!x || !global_amax || !packed_row || !scales_row || !packed_col || !scales_col)
    return NVFP4_E_NULL;
  if (!aligned(x, 16) || !aligned(packed_row, 8) || !aligned(packed_col, 8) ||
      !aligned(global_amax, 4))
    return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_rowcol(x, dt == NVFP4_BF16, M, K, global_amax, four_over_six,
                                         err == NVFP4_MSE, bound, packed_row, scales_row,
                                         packed_col, scales_col, stream));
}

nvfp4_status nvfp4_quantize_4over6_2d(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                      const float* global_amax, nvfp4_err err, float bound,
                                      uint8_t* packed_row, uint8_t* packed_col,
                                      uint8_t* tile_scales, void* stream) {
  if (nvfp4_status st = check_shape(M, K, true)) return st;
  if (!dtype_ok(dt)) return NVFP4_E_DTYPE;
  if (err != NVFP4_MAE && err != NVFP4_MSE) return NVFP4_E_ARG;
  if (!(bound == 256.0f || bound == 448.0f)) return NVFP4_E_ARG;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!x || !global_amax || !packed_row || !tile_scales) return NVFP4_E_NULL;
  if (!aligned(x, 16) || !aligned(packed_row, 8) || !aligned(packed_col, 8) ||
      !aligned(global_amax, 4))
    return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_4over6_2d(x, dt == NVFP4_BF16, M, K, global_amax,
                                            err == NVFP4_MSE, bound, packed_row, packed_col,
                                            tile_scales, stream));
}

nvfp4_status nvfp4_selftest_scan(int kind, uint32_t param, uint64_t first, uint64_t count,
                                 int chunk_log2, uint32_t* records, void* stream) {
  if (kind < 0 || kind > 4) return NVFP4_E_ARG;
  if (chunk_log2 < 0 || chunk_log2 > 24) return NVFP4_E_ARG;
  const uint64_t kPatterns = uint64_t(1) << 32;
  if (first > kPatterns || count > kPatterns - first) return NVFP4_E_RANGE;
  if ((kind == 3 || kind == 4) && first + count > 256) return NVFP4_E_RANGE;
  if (count == 0) return NVFP4_OK;
  const uint64_t nchunks = (count + (uint64_t(1) << chunk_log2) - 1) >> chunk_log2;
  if (nchunks > (uint64_t(1) << 22)) return NVFP4_E_ARG;
  if (!records) return NVFP4_E_NULL;
  if (!aligned(records, 16)) return NVFP4_E_ALIGN;
  return hip_status(nvfp4::launch_selftest_scan(kind, param, first, count, chunk_log2, records, stream));
}

nvfp4_status nvfp4_selftest_launch_plan(int entry, int64_t M, int64_t K, int in_bf16, int variant,
                                        int64_t* plan) {
  if (entry < 0 || entry > 6) return NVFP4_E_ARG;
  const bool tiles = entry == 3 || entry == 4 || entry == 5 || (entry == 1 && variant == 1);
  if (nvfp4_status st = check_shape(M, K, tiles)) return st;
  if (!plan) return NVFP4_E_NULL;
  nvfp4::LaunchPlan p{};
  switch (entry) {
    case 0: p = nvfp4::plan_quant1x16(M, K); break;
    case 1: p = nvfp4::plan_dequant(M, K); break;
    case 2: p = nvfp4::plan_4over6(in_bf16 != 0, M, K); break;
    case 3: p = nvfp4::plan_quant2d(M, K); break;
    case 4: p = nvfp4::plan_rowcol(M, K, variant != 0); break;
    case 5: p = nvfp4::plan_4over6_2d(M, K, variant != 0); break;
    default: p = nvfp4::plan_amax(M, K, variant != 0); break;
  }
  plan[0] = p.kernel;
  plan[1] = p.launches;
  plan[2] = p.grid;
  plan[3] = p.block;
  return NVFP4_OK;
}

}  // extern "C"
