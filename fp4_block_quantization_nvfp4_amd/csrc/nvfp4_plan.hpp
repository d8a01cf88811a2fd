// Launch geometry of every kernel, computed on the host from the shape only.
// The launchers take their grids from these functions, and the test-support
// entry point nvfp4_selftest_launch_plan returns the same numbers, so a CPU
// test can check that every launch stays inside the dispatch limits (grid x
// workgroup size below 2^32 work-items) for every accepted shape.
#pragma once

#include <stdint.h>

namespace nvfp4 {

// Workgroup shapes (lanes; strips of 16 rows per workgroup for the 16x16 and
// row + column kernels).
constexpr int kThreads = 256;           // k_quant1x16, k_dequant: 4 lanes per 16-element block
constexpr int kRowThreads = 128;        // k_4over6_rows: one two-wave workgroup per row
constexpr int kRowMaxBlocks = kRowThreads * 8;  // longest row (in 16-element blocks) it takes
constexpr int64_t kRowChunk = int64_t(1) << 24;  // rows per k_4over6_rows launch
constexpr int k46MaxThreads = 1024;     // k_4over6 (generic): one workgroup per row
constexpr int64_t k46MaxGrid = int64_t(1) << 20;
constexpr int k2dThreads = 512;         // k_quant2d: columns covered by a workgroup
constexpr int kStrips = 16;
constexpr int kRowColThreads = 256, kRowColFosThreads = 128, kRowColStrips = 16, kRowColFosStrips = 16;
constexpr int k46TileThreads = 512, k46TileStrips = 16;
constexpr int kAmaxThreads = 256;
constexpr int kAmaxMaxGroups = 2048;
constexpr int64_t kAmaxRowGrid = 65536;

enum PlanKernel {
  PLAN_QUANT1X16 = 0,
  PLAN_DEQUANT = 1,
  PLAN_4OVER6_ROWS = 2,
  PLAN_4OVER6_GENERIC = 3,
  PLAN_QUANT2D = 4,
  PLAN_ROWCOL = 5,
  PLAN_4OVER6_2D = 6,
  PLAN_AMAX_PARTIAL = 7,
  PLAN_AMAX_ROWS = 8,
};

struct LaunchPlan {
  int kernel;        // PlanKernel
  int64_t launches;  // launches of that kernel (row chunks)
  int64_t grid;      // workgroups of the largest launch
  int block;         // lanes per workgroup
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// XCD-aware padded grid of the row + column and 16x16 kernels (a multiple
// of the 8 XCDs; padding workgroups exit at once).
inline int64_t xcd_grid(int64_t n) { return 8 * ceil_div(n, 8); }

inline LaunchPlan plan_quant1x16(int64_t M, int64_t K) {
  return {PLAN_QUANT1X16, 1, ceil_div(M * K / 4, kThreads), kThreads};
}

inline LaunchPlan plan_dequant(int64_t M, int64_t K) {
  return {PLAN_DEQUANT, 1, ceil_div(M * K / 4, kThreads), kThreads};
}

// bf16 rows of up to kRowMaxBlocks blocks take the row kernel, one workgroup
// per row and at most kRowChunk rows per launch; everything else the generic
// grid-stride kernel.
inline bool use_rows_kernel(int in_bf16, int64_t K) { return in_bf16 && K / 16 <= kRowMaxBlocks; }

inline LaunchPlan plan_4over6(int in_bf16, int64_t M, int64_t K) {
  if (use_rows_kernel(in_bf16, K))
    return {PLAN_4OVER6_ROWS, ceil_div(M, kRowChunk), M < kRowChunk ? M : kRowChunk, kRowThreads};
  int threads = (int)ceil_div(K / 16, 64) * 64;
  if (threads > k46MaxThreads) threads = k46MaxThreads;
  if (threads < 64) threads = 64;
  return {PLAN_4OVER6_GENERIC, 1, M < k46MaxGrid ? M : k46MaxGrid, threads};
}

inline int64_t quant2d_colgroups(int64_t K) { return ceil_div(K, k2dThreads); }
inline LaunchPlan plan_quant2d(int64_t M, int64_t K) {
  return {PLAN_QUANT2D, 1, quant2d_colgroups(K) * ceil_div(M / 16, kStrips), k2dThreads};
}

inline int rowcol_threads(int four_over_six) { return four_over_six ? kRowColFosThreads : kRowColThreads; }
inline int rowcol_strips(int four_over_six) { return four_over_six ? kRowColFosStrips : kRowColStrips; }
inline LaunchPlan plan_rowcol(int64_t M, int64_t K, int four_over_six) {
  const int nt = rowcol_threads(four_over_six);
  return {PLAN_ROWCOL, 1, xcd_grid(ceil_div(K, nt) * ceil_div(M / 16, rowcol_strips(four_over_six))), nt};
}

// Strips per workgroup of the 16x16 four-over-six kernel.  With columnwise
// output every workgroup takes k46TileStrips (each column's codes leave as
// one 128-byte segment).  Rowwise only, a shorter walk is taken when the
// grid would otherwise not give two workgroups per slot of the chip: the
// largest of 16, 8 and 4 strips with at least 1024 workgroups, else 4.
inline int tile_strips_4over6_2d(int64_t M, int64_t K, int columnwise) {
  if (columnwise) return k46TileStrips;
  const int64_t ncolg = ceil_div(K, k46TileThreads), nstrips = M / 16;
  for (int str = k46TileStrips; str > 4; str /= 2)
    if (ncolg * ceil_div(nstrips, str) >= 1024) return str;
  return 4;
}

inline LaunchPlan plan_4over6_2d(int64_t M, int64_t K, int columnwise) {
  const int str = tile_strips_4over6_2d(M, K, columnwise);
  return {PLAN_4OVER6_2D, 1, xcd_grid(ceil_div(K, k46TileThreads) * ceil_div(M / 16, str)), k46TileThreads};
}

inline int64_t amax_partial_groups(int64_t M, int64_t K) {
  int64_t g = ceil_div(M * K / 16, kAmaxThreads * 8);
  if (g < 1) g = 1;
  if (g > kAmaxMaxGroups) g = kAmaxMaxGroups;
  return g;
}
inline LaunchPlan plan_amax(int64_t M, int64_t K, int per_row) {
  if (per_row) return {PLAN_AMAX_ROWS, 1, M < kAmaxRowGrid ? M : kAmaxRowGrid, kAmaxThreads};
  return {PLAN_AMAX_PARTIAL, 1, amax_partial_groups(M, K), kAmaxThreads};
}

}  // namespace nvfp4
