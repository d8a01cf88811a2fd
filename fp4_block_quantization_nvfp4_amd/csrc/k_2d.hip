// Transposition-invariant 2D NVFP4 quantize: one e4m3 scale per 16x16 tile,
// shared by X and X^T, with round-to-nearest or stochastic rounding ("Stable
// FP4 Training via Transposition-Invariant Block Quantization", abstract).
// Rowwise codes [M, K/2] and the same codes transposed [K, M/2] are written in
// one pass (the fused row + column kernel the four-over-six pull request lists
// as a follow-up), so no caller-side transpose is needed.
//
// Mapping: a workgroup of 512 lanes (8 waves) covers 512 columns and walks
// down up to 16 strips of 16 rows (a 256 x 512 region).  In every strip wave w
// owns rows 2w and 2w + 1, and lane l of a wave holds columns 8l .. 8l + 7 of
// both rows, so one load instruction of a wave reads 1 KB (bf16) of one row:
// long contiguous runs per row, which the memory system streams much faster
// than 16 rows x 128 bytes.  Tile t of the strip (columns 16t .. 16t + 15) is
// the lane pair (2t, 2t + 1) of all eight waves: the tile amax is the max over
// the pair (one DPP swap), then over the eight waves through a small LDS
// table.  Strips are taken in groups of two with one barrier per group (one
// per strip: 7168x18432 SR 81.6 against 83.2 us); the table is
// double-buffered by group parity.  Codes come from the hardware fp32 -> e2m1 conversions:
// round-to-nearest (exact for finite inputs) or stochastic rounding with one
// 16-bit draw per element; tiles holding a NaN or an infinity use the
// software encoder.  The scale byte comes from the exact fp32 -> e4m3
// conversion.
//
// Outputs: each lane pair swaps one code word so that the even lane stores
// 8 bytes of row 2w and the odd lane 8 bytes of row 2w + 1 (each wave store
// covers 256 contiguous bytes of both rows).  A lane's two rows make one code
// byte for each of its eight columns (row 2w low nibble, row 2w + 1 high): the
// byte goes to LDS, into the column's 128-byte segment (16 strips x 8 bytes),
// and after the last strip 16 lanes per column write whole segments.  The
// 8-byte words of a column's segment are rotated by the writing lane's index,
// which spreads the byte writes of a wave over the LDS banks.  The next group
// of strips is prefetched into registers while the current one is encoded,
// with nontemporal loads (the input is read once; round-to-nearest 84.8 -> 71.5
// us at 7168x18432 bf16 against plain loads).
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"
#include "nvfp4_plan.hpp"
#include "nvfp4_strip.hpp"

namespace nvfp4 {

constexpr int k2dTiles = kStripTiles;
constexpr int k2dWaves = kStripWaves;
static_assert(k2dThreads == kStripLanes && kStrips == kStripCount, "strip geometry");
// strips whose tile amaxes are exchanged under one workgroup barrier; the
// next group is loaded while one is encoded
constexpr int k2dGroup = 2;

// Software codes of eight elements (any input; a NaN encodes +6, code 0x7),
// round-to-nearest or stochastic with draws from the pcg words of their four
// pairs (p0 a multiple of four).
template <bool SR>
NV_DEV uint32_t encode8_sw(const float x[8], float rho, uint32_t p0, const PcgGroup<4>& pq) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (SR) pcg_group(pq, p0, w);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = fabsf(x[i]) * rho;
    float q;
    uint32_t mag;
    if (SR) mag = e2m1_sr(v, (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu, q);
    else mag = e2m1_rtn(v, q);
    const uint32_t neg = (v != v) ? 0u : (f2bits(x[i]) >> 31);
    c |= (mag | (neg << 3)) << (4 * i);
  }
  return c;
}

// Hardware codes of eight finite-or-infinite elements (pair index p0 of the
// first two, a multiple of four, for the draws).
template <bool SR>
NV_DEV uint32_t encode8_hw(const float x[8], float rho, uint32_t p0, const PcgGroup<4>& pq) {
  if (SR) {
    uint32_t nw[4];
    pcg_group(pq, p0, nw);
#pragma unroll
    for (int j = 0; j < 4; ++j) nw[j] = ~nw[j];
    return hw_fp4_sr_word(x, rho, nw);
  }
  uint32_t c = any_u32();
  c = hw_fp4_pair<0>(c, x[0] * rho, x[1] * rho);
  c = hw_fp4_pair<1>(c, x[2] * rho, x[3] * rho);
  c = hw_fp4_pair<2>(c, x[4] * rho, x[5] * rho);
  c = hw_fp4_pair<3>(c, x[6] * rho, x[7] * rho);
  return c;
}

template <typename InT, bool SR, bool GLOBAL, bool COL, bool UP>
__global__ __launch_bounds__(k2dThreads) void k_quant2d(
    const InT* __restrict__ x, const float* __restrict__ global_amax, uint32_t key, int64_t M,
    int64_t K, uint8_t* __restrict__ packed_row, uint8_t* __restrict__ packed_col,
    uint8_t* __restrict__ tile_scales, int64_t ncolg) {
  constexpr int kU4 = Row8<InT>::kU4;
  // tile amax exchange: [group parity][strip of the group][tile][wave] =
  // (NaN-dropped max bits, NaN seen)
  __shared__ __align__(16) uint2 red[2][k2dGroup][k2dTiles * k2dWaves];
  // column segments: [column][16 words of 8 bytes], word of strip st at (st + lane) & 15
  __shared__ uint2 colbuf[COL ? k2dThreads * kStrips : 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // Strip groups are taken from the bottom of the tensor up: the per-tensor
  // amax pass that precedes this one streams the tensor top to bottom, so
  // its most recently read (last-level-cache resident) rows come first here.
  const int64_t nsg = (M / 16 + kStrips - 1) / kStrips;
  const int64_t rsg = (int64_t)blockIdx.x / ncolg, cg = (int64_t)blockIdx.x - rsg * ncolg;
  const int64_t sg = nsg - 1 - rsg;
  const int64_t c0 = cg * k2dThreads + 8 * lane;  // first column of this lane
  const bool active = c0 < K;                     // uniform over the tile's lane pair
  const int64_t nstrips_total = M / 16;
  const int nst = (int)((nstrips_total - sg * kStrips) < kStrips ? (nstrips_total - sg * kStrips) : kStrips);
  const int64_t rowA0 = sg * kStrips * 16 + 2 * wv;  // row 2w of the first strip

  const PcgGroup<4> pq = pcg_group_key<4>(key);  // draw words, uniform over the grid
  float S_dec = 1.0f, mul = 0.0f;
  if (GLOBAL) {
    float S_enc;
    global_scales(global_amax[0], 2688.0f, S_enc, S_dec);
    mul = S_enc * (1.0f / 6.0f);
  }
  // encode reciprocals of all 127 scale codes (ordered before their first
  // use by the first strip's barrier)
  __shared__ float rhoT[128];
  if (threadIdx.x < 127) rhoT[threadIdx.x] = encode_reciprocal(e4m3_decode(threadIdx.x), S_dec);

  // Loads are unconditional (no branch, so no merge of old and new register
  // contents that would make the prefetch wait): a lane past the last column
  // reads the tensor's last 8 columns, and the load past the last strip reads
  // the tensor's first two rows' first 8 columns on every lane (a few cache
  // lines instead of a 16th of the input again).  Neither is stored.
  // Strips are loaded and encoded in order, so their addresses and pair
  // indices advance by a fixed step (no per-strip 64-bit multiplies).
  const int64_t cl = active ? c0 : K - 8;
  const InT* lp = x + rowA0 * K + cl;  // loads of the next strip to load
  auto load = [&](int st, uint4* d) {
    const InT* p = st < nst ? lp : x;
    lp += 16 * K;
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < kU4; ++i) {
      const u4v a = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p) + i);
      const u4v b = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p + K) + i);
      d[i] = make_uint4(a.x, a.y, a.z, a.w);
      d[kU4 + i] = make_uint4(b.x, b.y, b.z, b.w);
    }
  };

  // rowwise store and pair index of row A (a multiple of four, since K and c0
  // are multiples of eight) of the next strip to encode
  uint8_t* sp = packed_row + row_dst_offset(rowA0, K, c0, lane);
  uint32_t pA = (uint32_t)((rowA0 * K + c0) >> 1);
  // tile amax of one strip: lane pair, then (after the barrier) the eight
  // waves; rt is the strip's slot for the lane's tile
  auto amax_phase = [&](const uint4* cur, uint2* rt) {
    uint32_t nd = 0, fl = 0;
    if (active) lane_amax(cur, static_cast<const InT*>(nullptr), nd, fl);
    const uint32_t o = pair_swap(nd), f = pair_swap(fl);
    nd = o > nd ? o : nd;
    fl |= f;
    if ((lane & 1) == 0) rt[wv] = make_uint2(nd, fl);
  };
  auto encode_phase = [&](int st, const uint4* cur, const uint2* rt) {
    uint8_t* const dst = sp;
    const uint32_t pa = pA, pb = pA + (uint32_t)(K >> 1);
    sp += 8 * K;
    pA += (uint32_t)(8 * K);
    uint32_t nd = 0, fl = 0;
    {
      const uint4* r4 = reinterpret_cast<const uint4*>(rt);
#pragma unroll
      for (int i = 0; i < k2dWaves / 2; ++i) {
        const uint4 v = r4[i];
        nd = v.x > nd ? v.x : nd;
        nd = v.z > nd ? v.z : nd;
        fl |= v.y | v.w;
      }
    }
    if (!active) return;
    const bool special = fl != 0u || nd == 0x7F800000u;  // a NaN or an infinity in the tile
    const float a = bits2f(nd);
    float sigma = GLOBAL ? a * mul : div_guarded(a, 6.0f, 1.0f / 6.0f);
    sigma = fminf(sigma, kE4m3Max);
    uint32_t sc = hw_e4m3_pair(sigma, 0.0f) & 0xFFu;
    // truncation-free: smallest e4m3 value >= sigma (sc <= 0x7E here, where
    // the hardware decode equals e4m3_decode)
    if (UP && hw_e4m3_value<0>(sc) < sigma && sc < 0x7Eu) sc += 1u;
    const float rho = rhoT[sc];
    float xa[8], xb[8];
    widen8(cur, static_cast<const InT*>(nullptr), xa);
    widen8(cur + kU4, static_cast<const InT*>(nullptr), xb);
    uint32_t ca, cb;
    if (!special) {
      ca = encode8_hw<SR>(xa, rho, pa, pq);
      cb = encode8_hw<SR>(xb, rho, pb, pq);
    } else {
      ca = encode8_sw<SR>(xa, rho, pa, pq);
      cb = encode8_sw<SR>(xb, rho, pb, pq);
    }
    store_rows_pair(dst, lane, ca, cb);
    if (wv == 0 && (lane & 1) == 0)
      tile_scales[(sg * kStrips + st) * (K / 16) + c0 / 16] = (uint8_t)sc;
    if (COL) stage_col_bytes(colbuf, lane, wv, st, ca, cb);
  };

  // Two groups of register buffers: the next group of strips is loaded while
  // one is reduced and encoded.  The loop is unrolled by the two groups so
  // every buffer stays in fixed registers (no copies, which would wait for
  // the loads).  Group parity h alternates the tile amax slots, so a wave
  // that runs ahead never overwrites slots another wave still reads.
  constexpr int kRing = 2 * k2dGroup;
  uint4 raw[kRing][2 * kU4];
#pragma unroll
  for (int k = 0; k < k2dGroup; ++k) load(k, raw[k]);
  const int tslot = (lane >> 1) * k2dWaves;
  for (int st0 = 0; st0 < nst; st0 += kRing) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g0 = st0 + h * k2dGroup;  // first strip of the group
      if (g0 < nst) {
#pragma unroll
        for (int k = 0; k < k2dGroup; ++k) load(g0 + k2dGroup + k, raw[(1 - h) * k2dGroup + k]);
#pragma unroll
        for (int k = 0; k < k2dGroup; ++k) amax_phase(raw[h * k2dGroup + k], &red[h][k][tslot]);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < k2dGroup; ++k)
          if (g0 + k < nst) encode_phase(g0 + k, raw[h * k2dGroup + k], &red[h][k][tslot]);
      }
    }
  }
  if (COL) {
    __syncthreads();
    flush_col_segments(colbuf, cg, sg, nst, M, K, packed_col);
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
