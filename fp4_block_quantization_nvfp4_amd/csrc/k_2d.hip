// Transposition-invariant 2D NVFP4 quantize: one e4m3 scale per 16x16 tile,
// shared by X and X^T, with round-to-nearest or stochastic rounding ("Stable
// FP4 Training via Transposition-Invariant Block Quantization", abstract).
// Rowwise codes [M, K/2] and the same codes transposed [K, M/2] are written in
// one pass (the fused row + column kernel the four-over-six pull request lists
// as a follow-up), so no caller-side transpose is needed.
//
// Mapping: a workgroup of 512 lanes covers 512 columns and walks down up to
// 16 strips of 16 rows (a 256 x 512 region); in each strip it holds 32 tiles
// side by side, four per wave.  Lane (t, r) = (tid / 16, tid % 16)
// holds row r of tile t: 16 consecutive elements read with 128-bit loads, so
// each wave reads 16 rows x 128 contiguous bytes.  The tile amax is reduced
// across the 16 lanes of the tile with cross-lane max (all 16 lanes of a tile
// sit in one 16-lane row of the wave; DPP, no LDS).  Codes come from the
// hardware fp32 -> e2m1 conversions: round-to-nearest (exact for finite
// inputs) or stochastic rounding with one 16-bit draw per element; tiles
// holding a NaN or an infinity use the software encoder.  The scale byte
// comes from the exact fp32 -> e4m3 conversion.  The rowwise codes go out as
// one 8-byte store per lane.  For the columnwise codes each lane stages its
// 16 codes as bytes in LDS; lane (t, c) then gathers column c of its tile
// into a per-column buffer that is written out once per workgroup.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"
#include "nvfp4_plan.hpp"

namespace nvfp4 {

constexpr int k2dTiles = k2dThreads / 16;   // tiles side by side

// Max over the 16 lanes of a DPP row (every lane of the row gets it): two
// quad permutations, then the half-row and row mirrors.
NV_DEV uint32_t row16_max_u32(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false);
  return o > v ? o : v;
}

constexpr int kColStride = kStrips + 1;  // uint2 per column in the column buffer (+1 spreads banks)

template <typename InT, bool SR, bool GLOBAL, bool COL, bool UP>
__global__ __launch_bounds__(k2dThreads) void k_quant2d(
    const InT* __restrict__ x, const float* __restrict__ global_amax, uint32_t key, int64_t M,
    int64_t K, uint8_t* __restrict__ packed_row, uint8_t* __restrict__ packed_col,
    uint8_t* __restrict__ tile_scales, int64_t ncolg) {
  __shared__ uint4 stage[k2dTiles * 17];  // per tile 16 rows of 16 code bytes, tile stride 17 (bank spread)
  __shared__ uint2 colbuf[COL ? k2dThreads * kColStride : 1];
  const int t = threadIdx.x >> 4, r = threadIdx.x & 15;
  // Strip groups are taken from the bottom of the tensor up: the per-tensor
  // amax pass that precedes this one streams the tensor top to bottom, so
  // its most recently read (last-level-cache resident) rows come first here.
  const int64_t nsg = (M / 16 + kStrips - 1) / kStrips;
  const int64_t rsg = (int64_t)blockIdx.x / ncolg, cg = (int64_t)blockIdx.x - rsg * ncolg;
  const int64_t sg = nsg - 1 - rsg;
  const int64_t col0 = cg * k2dThreads + 16 * t;
  const bool active = col0 < K;  // uniform over the 16 lanes of a tile
  const int64_t nstrips_total = M / 16;
  const int nst = (int)((nstrips_total - sg * kStrips) < kStrips ? (nstrips_total - sg * kStrips) : kStrips);

  float S_dec = 1.0f, mul = 0.0f;
  if (GLOBAL) {
    float S_enc;
    global_scales(global_amax[0], 2688.0f, S_enc, S_dec);
    mul = S_enc * (1.0f / 6.0f);
  }

  // The next strip's 16 elements are loaded while the current one is
  // encoded (two register buffers of raw input).
  constexpr int kRaw = sizeof(InT) * 16 / 16;  // uint4 per 16 elements
  uint4 nxt[kRaw];
  if (active) {
    const uint4* p = reinterpret_cast<const uint4*>(x + (sg * kStrips * 16 + r) * K + col0);
#pragma unroll
    for (int i = 0; i < kRaw; ++i) nxt[i] = p[i];
  }
  for (int st = 0; st < nst; ++st) {
    const int64_t row0 = (sg * kStrips + st) * 16;
    const int64_t row = row0 + r;
    uint4 cur[kRaw];
#pragma unroll
    for (int i = 0; i < kRaw; ++i) cur[i] = nxt[i];
    if (active && st + 1 < nst) {
      const uint4* p = reinterpret_cast<const uint4*>(x + (row + 16) * K + col0);
#pragma unroll
      for (int i = 0; i < kRaw; ++i) nxt[i] = p[i];
    }
    float xv[16];
    uint32_t ab = 0;  // magnitude bit patterns: integer max = value max; >= 0x7F800000 flags NaN/inf
    if (active) {
      load16(reinterpret_cast<const InT*>(cur), xv);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t m = f2bits(xv[i]) & 0x7FFFFFFFu;
        ab = m > ab ? m : ab;
      }
    }
    ab = row16_max_u32(ab);
    const bool special = ab >= 0x7F800000u;
    float a = bits2f(ab);
    if (special) {  // NaN-dropping tile amax (all 16 lanes of the tile take this branch)
      float l = 0.0f;
      if (active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) l = fmaxf(l, abs_nan0(xv[i]));
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) l = fmaxf(l, __shfl_xor(l, off, 64));
      a = l;
    }

    uint32_t c0 = 0, c1 = 0;
    if (active) {
      float sigma = GLOBAL ? a * mul : div_guarded(a, 6.0f, 1.0f / 6.0f);
      sigma = fminf(sigma, kE4m3Max);
      uint32_t sc = hw_e4m3_pair(sigma, 0.0f) & 0xFFu;
      float s = e4m3_decode(sc);
      if (UP && s < sigma && sc < 0x7Eu) {  // truncation-free: smallest e4m3 value >= sigma
        sc += 1u;
        s = e4m3_decode(sc);
      }
      const float rho = encode_reciprocal(s, S_dec);
      if (SR && !special) {
        // stochastic rounding by the hardware conversion, one draw per element
        const uint32_t p0 = (uint32_t)((row * K + col0) >> 1);
        uint32_t nw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) nw[j] = ~pcg_hash((p0 + j) ^ key);
        c0 = hw_fp4_sr_word(xv, rho, nw);
        c1 = hw_fp4_sr_word(xv + 8, rho, nw + 4);
      } else if (!SR && !special) {
        c0 = hw_fp4_pair<0>(c0, xv[0] * rho, xv[1] * rho);
        c0 = hw_fp4_pair<1>(c0, xv[2] * rho, xv[3] * rho);
        c0 = hw_fp4_pair<2>(c0, xv[4] * rho, xv[5] * rho);
        c0 = hw_fp4_pair<3>(c0, xv[6] * rho, xv[7] * rho);
        c1 = hw_fp4_pair<0>(c1, xv[8] * rho, xv[9] * rho);
        c1 = hw_fp4_pair<1>(c1, xv[10] * rho, xv[11] * rho);
        c1 = hw_fp4_pair<2>(c1, xv[12] * rho, xv[13] * rho);
        c1 = hw_fp4_pair<3>(c1, xv[14] * rho, xv[15] * rho);
      } else {
        uint32_t w[8];
        if (SR) {
          const uint32_t p0 = (uint32_t)((row * K + col0) >> 1);
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = pcg_hash((p0 + j) ^ key);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = fabsf(xv[i]) * rho;
          float q;
          uint32_t mag;
          if (SR) mag = e2m1_sr(v, (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu, q);
          else mag = e2m1_rtn(v, q);
          const uint32_t neg = (v != v) ? 0u : (f2bits(xv[i]) >> 31);
          const uint32_t code = mag | (neg << 3);
          if (i < 8) c0 |= code << (4 * i);
          else c1 |= code << (4 * (i - 8));
        }
      }
      *reinterpret_cast<uint2*>(packed_row + row * (K / 2) + col0 / 2) = make_uint2(c0, c1);
      if (r == 0) tile_scales[(row0 / 16) * (K / 16) + col0 / 16] = (uint8_t)sc;
    }
    if (COL) {
      // Stage the 16 codes of this tile row one per byte; lane (t, c) then
      // gathers column c of its tile (rows 0..15, two codes per byte in row
      // order) into the column buffer slot of this strip.
      if (active) {
        stage[17 * t + r] = make_uint4(
            (c0 & 0xFu) | ((c0 >> 4) & 0xFu) << 8 | ((c0 >> 8) & 0xFu) << 16 | ((c0 >> 12) & 0xFu) << 24,
            ((c0 >> 16) & 0xFu) | ((c0 >> 20) & 0xFu) << 8 | ((c0 >> 24) & 0xFu) << 16 | ((c0 >> 28) & 0xFu) << 24,
            (c1 & 0xFu) | ((c1 >> 4) & 0xFu) << 8 | ((c1 >> 8) & 0xFu) << 16 | ((c1 >> 12) & 0xFu) << 24,
            ((c1 >> 16) & 0xFu) | ((c1 >> 20) & 0xFu) << 8 | ((c1 >> 24) & 0xFu) << 16 | ((c1 >> 28) & 0xFu) << 24);
      }
      __syncthreads();
      if (active) {
        const uint8_t* tile = reinterpret_cast<const uint8_t*>(&stage[17 * t]);
        const int c = r;
        uint32_t o0 = 0, o1 = 0;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const uint32_t code = tile[16 * rr + c];
          if (rr < 8) o0 |= code << (4 * rr);
          else o1 |= code << (4 * (rr - 8));
        }
        colbuf[(16 * t + c) * kColStride + st] = make_uint2(o0, o1);
      }
      __syncthreads();
    }
  }
  if (COL) {
    // Each column of this workgroup owns nst * 8 contiguous bytes of its
    // packed_col row; 16 lanes write one column (8 bytes each), so every
    // store instruction covers four whole column segments.
    const int q = threadIdx.x & 15;
    for (int cc = threadIdx.x >> 4; cc < k2dThreads; cc += k2dThreads / 16) {
      const int64_t col = cg * k2dThreads + cc;
      if (col < K && q < nst)
        *reinterpret_cast<uint2*>(packed_col + col * (M / 2) + sg * (kStrips * 8) + q * 8) =
            colbuf[cc * kColStride + q];
    }
  }
}

template <typename InT, bool SR, bool GLOBAL, bool UP>
static int launch2d_col(const InT* x, const float* ga, uint32_t key, int64_t M, int64_t K,
                        uint8_t* pr, uint8_t* pc, uint8_t* ts, hipStream_t st) {
  const int64_t ncolg = quant2d_colgroups(K);
  const LaunchPlan pl = plan_quant2d(M, K);
  const dim3 grid((unsigned)pl.grid), block(pl.block);
  if (pc) hipLaunchKernelGGL((k_quant2d<InT, SR, GLOBAL, true, UP>), grid, block, 0, st, x, ga, key, M, K, pr, pc, ts, ncolg);
  else hipLaunchKernelGGL((k_quant2d<InT, SR, GLOBAL, false, UP>), grid, block, 0, st, x, ga, key, M, K, pr, pc, ts, ncolg);
  return (int)hipGetLastError();
}

template <typename InT, bool UP>
static int launch2d_typed(const InT* x, const float* ga, int sr, uint32_t key, int64_t M,
                          int64_t K, uint8_t* pr, uint8_t* pc, uint8_t* ts, hipStream_t st) {
  if (sr && ga) return launch2d_col<InT, true, true, UP>(x, ga, key, M, K, pr, pc, ts, st);
  if (sr) return launch2d_col<InT, true, false, UP>(x, ga, key, M, K, pr, pc, ts, st);
  if (ga) return launch2d_col<InT, false, true, UP>(x, ga, key, M, K, pr, pc, ts, st);
  return launch2d_col<InT, false, false, UP>(x, ga, key, M, K, pr, pc, ts, st);
}

template <typename InT>
static int launch2d_round(const InT* x, const float* ga, int sr, uint32_t key, int round_up,
                          int64_t M, int64_t K, uint8_t* pr, uint8_t* pc, uint8_t* ts,
                          hipStream_t st) {
  if (round_up) return launch2d_typed<InT, true>(x, ga, sr, key, M, K, pr, pc, ts, st);
  return launch2d_typed<InT, false>(x, ga, sr, key, M, K, pr, pc, ts, st);
}

int launch_quant2d(const void* x, int in_bf16, int64_t M, int64_t K, const float* global_amax,
                   int sr, uint32_t seed, uint32_t step, int round_up, uint8_t* packed_row,
                   uint8_t* packed_col, uint8_t* tile_scales, void* stream) {
  if (M == 0 || K == 0) return 0;
  const uint32_t key = rng_key_host(seed, step);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (in_bf16)
    return launch2d_round(reinterpret_cast<const uint16_t*>(x), global_amax, sr, key, round_up, M,
                          K, packed_row, packed_col, tile_scales, st);
  return launch2d_round(reinterpret_cast<const float*>(x), global_amax, sr, key, round_up, M, K,
                        packed_row, packed_col, tile_scales, st);
}

}  // namespace nvfp4
