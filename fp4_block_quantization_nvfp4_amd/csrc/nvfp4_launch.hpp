// Host-side launchers of the NVFP4 kernels.  Arguments are already validated
// by the C ABI layer (api.cpp); each launcher returns a hipError_t as int.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// dtype codes match nvfp4_dtype: 0 fp32, 1 bf16.  out_kind: 0 none, 1 bf16, 2 fp32.
int launch_quant1x16(const void* x, int in_bf16, int64_t M, int64_t K, float* residual,
                     const float* global_amax, int sr, uint32_t seed, uint32_t step,
                     uint8_t* packed, uint8_t* scales, void* out, int out_kind, void* stream);

// scale_mode: 0 none, 1 tensor, 2 row.  out_bf16: 1 bf16, 0 fp32.
int launch_dequant(const uint8_t* packed, const uint8_t* scales, int64_t M, int64_t K,
                   int tile16, const float* global_amax, int scale_mode, float bound,
                   void* out, int out_bf16, void* stream);

// mode: 1 tensor, 2 row.  amax_is_input: row amax read (1) or computed in-pass (0).
int launch_4over6(const void* x, int in_bf16, int64_t M, int64_t K, float* amax, int mode,
                  int amax_is_input, int mse, float bound, uint8_t* packed, uint8_t* scales,
                  void* stream);

int launch_quant2d(const void* x, int in_bf16, int64_t M, int64_t K, const float* global_amax,
                   int sr, uint32_t seed, uint32_t step, int round_up, uint8_t* packed_row,
                   uint8_t* packed_col, uint8_t* tile_scales, void* stream);

int launch_rowcol(const void* x, int in_bf16, int64_t M, int64_t K, const float* global_amax,
                  int four_over_six, int mse, float bound, uint8_t* packed_row,
                  uint8_t* scales_row, uint8_t* packed_col, uint8_t* scales_col, void* stream);

int launch_4over6_2d(const void* x, int in_bf16, int64_t M, int64_t K, const float* global_amax,
                     int mse, float bound, uint8_t* packed_row, uint8_t* packed_col,
                     uint8_t* tile_scales, void* stream);

size_t amax_workspace_bytes(int64_t M, int64_t K);
// mode: 1 tensor (two passes through workspace), 2 row.
int launch_amax(const void* x, int in_bf16, int64_t M, int64_t K, const float* residual,
                int mode, float* amax_out, void* workspace, void* stream);

// Allocation-free per-tensor / per-row amax: partials in the library's own
// device scratch array (k_amax.hip).
int64_t amax_noalloc_max_partials();
int launch_amax_noalloc(const void* x, int in_bf16, int64_t M, int64_t K, const float* residual,
                        int mode, float* amax_out, void* stream);

// Test support: exhaustive conversion scans (k_selftest.hip).
int launch_selftest_scan(int kind, uint32_t param, uint64_t first, uint64_t count, int chunk_log2,
                         uint32_t* records, void* stream);

}  // namespace nvfp4
