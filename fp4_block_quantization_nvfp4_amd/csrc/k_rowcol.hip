// Two kernels that produce the forward (rowwise) and the transposed
// (columnwise) NVFP4 operands of one tensor in a single pass over it, with
// one per-tensor global amax and round-to-nearest:
//
//  * k_rowcol - 1x16 blocks along K for X and, independently, 1x16 blocks
//    along M (16 consecutive rows of one column) for X^T, each block with its
//    own scale: the standard encode (sigma = a * (S_enc * (1/6)), bound 448)
//    or four-over-six (bound 256 or 448).  This is the fused row + column
//    kernel that the four-over-six pull request lists among its follow-up
//    fusions, replacing a caller-side transpose and second quantize for the
//    backward operands.
//  * k_4over6_2d - four-over-six on 16x16 tiles: one scale per tile, shared
//    by X and X^T (transposition-invariant paper, abstract); each tile row
//    sums its 16 errors in element order, the 16 row sums are combined by the
//    exact width-16 tree of the pull request's CuTe DSL kernel Design, and
//    map-to-4 is kept iff its tile error is strictly lower.
//
// Mapping (both): a workgroup of NT lanes covers NT columns and walks down
// up to STR strips of 16 rows (256 x 16 for the standard k_rowcol, 128 x 16
// for its four-over-six form, 512 x 16 for k_4over6_2d); in a strip it holds
// NT / 16 tiles side by side, and each lane reads 16 consecutive elements of
// one row (128-bit loads; the next strip's row is loaded while the current
// one is encoded).  k_rowcol gives lane (r, t) = (tid / (NT / 16),
// tid % (NT / 16)) row r of tile t, so the NT / 16 lanes of a row read one
// contiguous NT-column run (512 bytes of bf16 for the standard form: a wave
// reads 4 rows x 512 bytes, which streams about 17% faster than 16 rows x 128
// bytes), then stages the tile's raw input in LDS, and lane (tc, c) =
// (tid / 16, tid % 16) encodes column c of tile tc.  k_4over6_2d keeps the
// 16 rows of a tile in one 16-lane row of a wave (lane (t, r) = (tid / 16,
// tid % 16)) for its cross-lane tile reductions and stages its codes (the
// same codes, transposed).  The columnwise codes and scales of each column
// are gathered in LDS across the strips and written out once per workgroup
// as whole column segments.
//
// Four-over-six: with A and D fixed for the tensor, the encode reciprocals
// and dequant values of every scale code are tabulated in LDS once per
// workgroup.  Blocks or tiles that hold a NaN or an infinity take the
// software encoder and true divisions.
#include "nvfp4_device.hpp"
#include "nvfp4_fos.hpp"
#include "nvfp4_launch.hpp"
#include "nvfp4_plan.hpp"

namespace nvfp4 {

// Workgroup shapes (nvfp4_plan.hpp: lanes = columns covered, 16-row strips
// per workgroup).  The four-over-six row + column pass is VALU-heavy and
// gains from more resident workgroups (128 columns: half the LDS); the
// standard pass is bound by its memory pattern and prefers 256-byte row
// segments.

// XCD-aware work order.  The dispatcher hands workgroup i to XCD i % 8, and
// each XCD has its own L2.  With a grid of xcd_grid(n) workgroups, XCD x
// takes work items x * ceil(n / 8) + 0, 1, 2, ... in dispatch order, so
// neighbouring items (which write the two halves of shared output lines)
// run in one L2.  Indices >= n are padding: such a workgroup exits at once.
// The kernels map item w to n - 1 - w, so the rows the per-tensor amax pass
// (top to bottom) read last, still in the last-level cache, are read first.
NV_DEV int64_t xcd_work_index(int64_t n) {
  return (int64_t)(blockIdx.x & 7u) * ((n + 7) / 8) + (int64_t)(blockIdx.x >> 3);
}

// Max over the 16 lanes of a DPP row (every lane of the row gets it).
NV_DEV uint32_t row16_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false);
  return o > v ? o : v;
}

// Value of lane i ^ 8, i ^ 4 (given a value already symmetric under ^ 8),
// i ^ 2 and i ^ 1 within a 16-lane DPP row: a rotation of the row by 8 is
// the ^ 8 exchange; after it a rotation by 4 delivers the partner i ^ 4's
// value (lanes i + 4 and i - 4 then hold equal values); the quad
// permutations [2,3,0,1] and [1,0,3,2] are ^ 2 and ^ 1.  Every lane of the
// row must be active.
NV_DEV uint32_t dpp_x8(uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false); }
NV_DEV uint32_t dpp_x4s(uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xF, 0xF, false); }
NV_DEV uint32_t dpp_x2(uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false); }
NV_DEV uint32_t dpp_x1(uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false); }

// Sum of the 16 lanes' values of a tile in the tree order
// ((g0+g8)+(g4+g12)) + ((g2+g10)+(g6+g14)) for the even lanes and the same
// over the odd lanes, then even + odd: exchanging with lane ^ 8, ^ 4, ^ 2,
// ^ 1 forms exactly these partial sums (fp addition is commutative, so both
// partners of an exchange hold the same bits) and every lane ends with the
// tile total.
NV_DEV float tree16_sum(float e) {
  e = e + bits2f(dpp_x8(f2bits(e)));
  e = e + bits2f(dpp_x4s(f2bits(e)));
  e = e + bits2f(dpp_x2(f2bits(e)));
  e = e + bits2f(dpp_x1(f2bits(e)));
  return e;
}

// True on every lane of a 16-lane tile iff f holds on all 16 of them.
NV_DEV bool all16(bool f) {
  uint32_t v = f ? 1u : 0u;
  v &= dpp_x8(v);
  v &= dpp_x4s(v);
  v &= dpp_x2(v);
  v &= dpp_x1(v);
  return v != 0u;
}

NV_DEV uint32_t absmax_bits16(const float v[16]) {
  uint32_t ab = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t m = f2bits(v[i]) & 0x7FFFFFFFu;
    ab = m > ab ? m : ab;
  }
  return ab;
}

NV_DEV float absmax_nan_drop16(const float v[16]) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, abs_nan0(v[i]));
  return a;
}

// Standard 1x16 block with a global scale: sigma = a * mul, mul =
// S_enc * (1/6); ab is the block's largest magnitude bit pattern (a NaN
// pattern tops it); returns the scale byte, codes in c.
NV_DEV uint32_t block_standard(const float v[16], uint32_t ab, float mul, float S_dec, uint32_t c[2]) {
  if (ab < 0x7F800000u) {
    const uint32_t sc = hw_e4m3_pair(fminf(bits2f(ab) * mul, kE4m3Max), 0.0f) & 0xFFu;
    encode16_hw(v, encode_reciprocal(e4m3_decode(sc), S_dec), c);
    return sc;
  }
  const uint32_t sc = e4m3_encode(fminf(absmax_nan_drop16(v) * mul, kE4m3Max));
  encode16_sw(v, encode_reciprocal(e4m3_decode(sc), S_dec), c);
  return sc;
}

// Raw input of 16 elements (uint4 words) and its conversion to fp32.
template <typename InT>
struct Raw16 {
  static constexpr int kWords = sizeof(InT);  // uint4 per 16 elements: 2 (bf16) or 4 (fp32)
  uint4 w[kWords];
  NV_DEV void load(const InT* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = q[i];
  }
  NV_DEV void to_f32(float v[16]) const { load16(reinterpret_cast<const InT*>(w), v); }
  // largest magnitude bit pattern as fp32 bits (bf16: one packed 16-bit max
  // per word); a NaN pattern tops it
  NV_DEV uint32_t absmax_bits() const {
    if constexpr (sizeof(InT) == 2) {
      typedef unsigned short us2 __attribute__((ext_vector_type(2)));
      const uint32_t u[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
      us2 m = __builtin_bit_cast(us2, u[0] & 0x7FFF7FFFu);
#pragma unroll
      for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, u[i] & 0x7FFF7FFFu));
      return (uint32_t)(m.x > m.y ? m.x : m.y) << 16;
    } else {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u[4] = {w[i].x & 0x7FFFFFFFu, w[i].y & 0x7FFFFFFFu, w[i].z & 0x7FFFFFFFu, w[i].w & 0x7FFFFFFFu};
#pragma unroll
        for (int j = 0; j < 4; ++j) m = u[j] > m ? u[j] : m;
      }
      return m;
    }
  }
};

// LDS staging of one 16x16 tile of raw input for the columnwise blocks:
// 16 rows of 16 elements, row stride kRow bytes, tile stride kTile bytes.
// bf16 rows are dense (32 B); fp32 rows are padded to 80 B.  The extra 32 or
// 64 bytes per tile put the four tiles of a wave in different bank windows
// when each lane reads down its column.
template <typename InT>
struct StageTile {
  static constexpr int kRow = sizeof(InT) == 2 ? 32 : 80;
  static constexpr int kTile = 16 * kRow + 16 * (int)sizeof(InT);
  NV_DEV static void put_row(uint8_t* tile, int r, const Raw16<InT>& raw) {
    uint4* d = reinterpret_cast<uint4*>(tile + r * kRow);
#pragma unroll
    for (int i = 0; i < Raw16<InT>::kWords; ++i) d[i] = raw.w[i];
  }

  NV_DEV static void get_col(const uint8_t* tile, int c, float v[16]) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      if constexpr (sizeof(InT) == 2)
        v[rr] = bits2f((uint32_t)*reinterpret_cast<const uint16_t*>(tile + rr * kRow + 2 * c) << 16);
      else
        v[rr] = *reinterpret_cast<const float*>(tile + rr * kRow + 4 * c);
    }
  }
};

// Write the column buffers of a workgroup: column cc of the workgroup owns
// nst * 8 contiguous code bytes of its packed_col row (and nst scale bytes of
// its scales_col row); 16 lanes serve one column.
template <int NT, int STR>
NV_DEV void flush_columns(const uint2* colbuf, const uint8_t* csbuf, int64_t cg, int64_t sg, int nst,
                          int64_t M, int64_t K, uint8_t* packed_col, uint8_t* scales_col) {
  const int q = threadIdx.x & 15;
  for (int cc = threadIdx.x >> 4; cc < NT; cc += NT / 16) {
    const int64_t col = cg * NT + cc;
    if (col < K && q < nst) {
      const int64_t strip = sg * STR + q;  // STR strips per workgroup
      *reinterpret_cast<uint2*>(packed_col + col * (M / 2) + strip * 8) = colbuf[cc * (STR + 1) + q];
      if (scales_col) scales_col[col * (M / 16) + strip] = csbuf[cc * (STR + 1) + q];
    }
  }
}

template <typename InT, bool FOS, bool MSE, int NT, int STR, bool RING = !FOS>
__global__ __launch_bounds__(NT) void k_rowcol(
    const InT* __restrict__ x, const float* __restrict__ global_amax, float D, int64_t M, int64_t K,
    uint8_t* __restrict__ packed_row, uint8_t* __restrict__ scales_row,
    uint8_t* __restrict__ packed_col, uint8_t* __restrict__ scales_col, int64_t ncolg) {
  // The raw input is staged (fp32 staging of the widened values would spare
  // the column pass its conversions, but the extra LDS cuts the resident
  // workgroups of the four-over-six form from 6 to 5 per CU: 121.7 ->
  // 143.1 us).
  using ST = StageTile<InT>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[(NT / 16) * ST::kTile];
  __shared__ uint2 colbuf[NT * (STR + 1)];
  __shared__ uint8_t csbuf[NT * (STR + 1)];
  __shared__ float rhoT[FOS ? 128 : 1];
  __shared__ float WT[FOS ? 128 : 1];  // W = s * S_dec per scale code
  // row pass: lane (r, t) holds row r of tile t, so the NT / 16 lanes of a
  // row read NT * sizeof(InT) contiguous bytes; column pass: lane (tc, c)
  // owns column c of tile tc
  const int t = threadIdx.x % (NT / 16), r = threadIdx.x / (NT / 16);
  const int tc = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int64_t nwork = ncolg * ((M / 16 + STR - 1) / STR);
  const int64_t w = xcd_work_index(nwork);
  if (w >= nwork) return;  // grid padding (uniform over the workgroup)
  // work items run from the bottom of the tensor up (see xcd_work_index)
  const int64_t wr = nwork - 1 - w;
  const int64_t sg = wr / ncolg, cg = wr - sg * ncolg;
  const int64_t col0 = cg * NT + 16 * t;
  const bool active = col0 < K;              // row pass
  const bool active_c = cg * NT + 16 * tc < K;  // column pass
  const int64_t nstrips = M / 16;
  const int nst = (int)((nstrips - sg * STR) < STR ? (nstrips - sg * STR) : STR);

  const float A = global_amax[0];
  float S_enc, S_dec;
  global_scales(A, D, S_enc, S_dec);
  const float mul = S_enc * (1.0f / 6.0f);
  const bool lean = FOS && fos_row_in_range(A, S_dec);
  if (FOS) {
    if (threadIdx.x < 127) {
      const float s = e4m3_decode(threadIdx.x);
      rhoT[threadIdx.x] = encode_reciprocal(s, S_dec);
      WT[threadIdx.x] = s * S_dec;
    }
    __syncthreads();
  }

  // Loads are unconditional (a lane past the last column reads the row's last
  // 16 elements, the load past the last strip reads the tensor's first 16),
  // and a ring of two register buffers, with the loop unrolled by two, keeps
  // them in fixed registers: no merge of old and new contents, which would
  // make the next strip's prefetch wait before the current one is encoded.
  const InT* lp = x + (sg * STR * 16 + r) * K + (active ? col0 : K - 16);
  auto load = [&](int st, Raw16<InT>& d) {
    d.load(st < nst ? lp : x);
    lp += 16 * K;
  };
  auto body = [&](int st, const Raw16<InT>& cur) {
    const int64_t row = (sg * STR + st) * 16 + r;
    if (active) {
      float v[16];
      cur.to_f32(v);
      uint32_t rc[2];
      const uint32_t ab = cur.absmax_bits();
      const uint32_t sc = FOS ? fos_block_ab<MSE, true, true>(v, ab, lean, S_enc, S_dec, A, D, rhoT, rc, WT)
                              : block_standard(v, ab, mul, S_dec, rc);
      *reinterpret_cast<uint2*>(packed_row + row * (K / 2) + col0 / 2) = make_uint2(rc[0], rc[1]);
      scales_row[row * (K / 16) + col0 / 16] = (uint8_t)sc;
      ST::put_row(xs + t * ST::kTile, r, cur);
    }
    __syncthreads();
    if (active_c) {
      // lane (tc, c) owns column c of tile tc: rows 0..15 in order
      float v[16];
      ST::get_col(xs + tc * ST::kTile, c, v);
      uint32_t cc[2];
      const uint32_t sc = FOS ? fos_block_f32<MSE, true, true>(v, lean, S_enc, S_dec, A, D, rhoT, cc, WT)
                              : block_standard(v, absmax_bits16(v), mul, S_dec, cc);
      colbuf[(16 * tc + c) * (STR + 1) + st] = make_uint2(cc[0], cc[1]);
      csbuf[(16 * tc + c) * (STR + 1) + st] = (uint8_t)sc;
    }
    __syncthreads();
  };
  if constexpr (RING) {
    Raw16<InT> ring[2];
    load(0, ring[0]);
    for (int st0 = 0; st0 < nst; st0 += 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (st0 + k < nst) {
          load(st0 + k + 1, ring[k ^ 1]);
          body(st0 + k, ring[k]);
        }
      }
    }
  } else {
    Raw16<InT> nxt;
    load(0, nxt);
    for (int st = 0; st < nst; ++st) {
      const Raw16<InT> cur = nxt;
      load(st + 1, nxt);
      body(st, cur);
    }
  }
  flush_columns<NT, STR>(colbuf, csbuf, cg, sg, nst, M, K, packed_col, scales_col);
}

// str: strips per workgroup (STR with columnwise output, at most STR
// rowwise only; tile_strips_4over6_2d).
template <typename InT, bool MSE, bool COL, int NT, int STR>
__global__ __launch_bounds__(NT) void k_4over6_2d(
    const InT* __restrict__ x, const float* __restrict__ global_amax, float D, int64_t M, int64_t K,
    uint8_t* __restrict__ packed_row, uint8_t* __restrict__ packed_col,
    uint8_t* __restrict__ tile_scales, int64_t ncolg, int str) {
  __shared__ float rhoT[128];
  __shared__ uint2 colbuf[COL ? NT * (STR + 1) : 1];
  const int t = threadIdx.x >> 4, r = threadIdx.x & 15;
  const int64_t nwork = ncolg * ((M / 16 + str - 1) / str);
  const int64_t w = xcd_work_index(nwork);
  if (w >= nwork) return;  // grid padding (uniform over the workgroup)
  // work items run from the bottom of the tensor up (see xcd_work_index)
  const int64_t wr = nwork - 1 - w;
  const int64_t sg = wr / ncolg, cg = wr - sg * ncolg;
  const int64_t col0 = cg * NT + 16 * t;
  const bool active = col0 < K;
  const int64_t nstrips = M / 16;
  const int nst = (int)((nstrips - sg * str) < str ? (nstrips - sg * str) : str);

  const float A = global_amax[0];
  float S_enc, S_dec;
  global_scales(A, D, S_enc, S_dec);
  if (threadIdx.x < 127) rhoT[threadIdx.x] = encode_reciprocal(e4m3_decode(threadIdx.x), S_dec);
  __syncthreads();

  // unconditional loads (as in k_rowcol); the body is too large to unroll
  const InT* lp = x + (sg * str * 16 + r) * K + (active ? col0 : K - 16);
  auto load = [&](int st, Raw16<InT>& d) {
    d.load(st < nst ? lp : x);
    lp += 16 * K;
  };
  auto body = [&](int st, const Raw16<InT>& cur) {
    const int64_t row0 = (sg * str + st) * 16;
    const int64_t row = row0 + r;
    float v[16];
    uint32_t ab = 0;
    if (active) {
      cur.to_f32(v);
      ab = cur.absmax_bits();
    }
    ab = row16_max(ab);
    // NaN-dropping tile amax (the integer max of the magnitude bits is the
    // value max unless the tile holds a NaN)
    float a = bits2f(ab);
    if (ab > 0x7F800000u) {
      float l = active ? absmax_nan_drop16(v) : 0.0f;
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) l = fmaxf(l, __shfl_xor(l, off, 64));
      a = l;
    }
    const float sig6 = div_guarded(a, 6.0f, 1.0f / 6.0f) * S_enc;
    const uint32_t kk = hw_e4m3_pair(fminf(sig6, kE4m3Max), fminf(sig6 * 1.5f, kE4m3Max)) & 0x7F7Fu;
    const uint32_t k6 = kk & 0xFFu, k4 = kk >> 8;
    const float rho6 = rhoT[k6], rho4 = rhoT[k4];
    const float s6 = e4m3_decode(k6), s4 = e4m3_decode(k4);
    uint32_t c6[2] = {0u, 0u}, c4[2] = {0u, 0u};
    float E6 = 0.0f, E4 = 0.0f;
    if (active) {
      float v6[16], v4[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v6[i] = v[i] * rho6;
        v4[i] = v[i] * rho4;
      }
      encode16_hw(v, rho6, c6);
      encode16_hw(v, rho4, c4);
      E6 = approx_error16<MSE>(v6, c6);
      E4 = approx_error16<MSE>(v4, c4);
    }
    // the decision is uniform over the tile (every lane holds the same tree totals)
    int pick = certified_pick<MSE, 8>(tree16_sum(E6), tree16_sum(E4), s6 * S_dec, s4 * S_dec, a);
    // an undecided tile whose rows all have identical dequant values under
    // both candidates (same_dequant16) is an exact tie: map-to-6
    if (pick == -1 && all16(active && same_dequant16(c6, c4, s6, s4))) pick = 0;
    if (pick < 0) {  // exact row errors, then the same tree
      if (active) {
        if (pick == -1) {
          const float rD = recip_in_place(D);
          E6 = exact_error16<MSE>(v, c6, s6, A, D, rD);
          E4 = exact_error16<MSE>(v, c4, s4, A, D, rD);
        } else {
          E6 = candidate<MSE>(v, s6, rho6, A, D, c6[0], c6[1]);
          E4 = candidate<MSE>(v, s4, rho4, A, D, c4[0], c4[1]);
        }
      }
      E6 = tree16_sum(E6);
      E4 = tree16_sum(E4);
      pick = E4 < E6 ? 1 : 0;
    }
    const bool pick4 = pick == 1;
    const uint32_t c0 = pick4 ? c4[0] : c6[0], c1 = pick4 ? c4[1] : c6[1];
    if (active) {
      *reinterpret_cast<uint2*>(packed_row + row * (K / 2) + col0 / 2) = make_uint2(c0, c1);
      if (r == 0) tile_scales[(row0 / 16) * (K / 16) + col0 / 16] = (uint8_t)(pick4 ? k4 : k6);
    }
    if (COL) {
      // Column codes: rows 2k and 2k + 1 of the tile (lanes r = 2k, 2k + 1,
      // a DPP quad pair) make byte k of each column's strip word; the even
      // lane writes the bytes of columns 0..7, the odd lane those of 8..15.
      // The column buffer is written out once after the last strip, so no
      // barrier is needed here.
      const uint32_t p0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)c0, 0xB1, 0xF, 0xF, false);
      const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)c1, 0xB1, 0xF, 0xF, false);
      if (active) {
        const bool odd = r & 1;
        const uint32_t lo = odd ? p1 : c0;  // row 2k, this lane's eight columns
        const uint32_t hi = odd ? c1 : p0;  // row 2k + 1
        const uint32_t ev = (lo & 0x0F0F0F0Fu) | ((hi << 4) & 0xF0F0F0F0u);  // columns 0, 2, 4, 6
        const uint32_t od = ((lo >> 4) & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u);  // columns 1, 3, 5, 7
        uint8_t* cb = reinterpret_cast<uint8_t*>(colbuf) + ((16 * t + (odd ? 8 : 0)) * (STR + 1) + st) * 8 + (r >> 1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          cb[(2 * k) * (STR + 1) * 8] = (uint8_t)(ev >> (8 * k));
          cb[(2 * k + 1) * (STR + 1) * 8] = (uint8_t)(od >> (8 * k));
        }
      }
    }
  };
  Raw16<InT> nxt;
  load(0, nxt);
  for (int st = 0; st < nst; ++st) {
    const Raw16<InT> cur = nxt;
    load(st + 1, nxt);
    body(st, cur);
  }
  if (COL) {
    __syncthreads();
    flush_columns<NT, STR>(colbuf, nullptr, cg, sg, nst, M, K, packed_col, nullptr);
  }
}


template <typename InT>
static int launch_rowcol_t(const InT* x, const float* ga, int fos, int mse, float D, int64_t M,
                           int64_t K, uint8_t* pr, uint8_t* sr, uint8_t* pc, uint8_t* sc,
                           hipStream_t st) {
  int64_t ncolg;
  const LaunchPlan pl = plan_rowcol(M, K, fos);
  const dim3 grid((unsigned)pl.grid), block(pl.block);
  if (!fos) {
    constexpr int NT = kRowColThreads, STR = kRowColStrips;
    ncolg = ceil_div(K, NT);
    hipLaunchKernelGGL((k_rowcol<InT, false, false, NT, STR>), grid, block, 0, st, x, ga, D, M, K, pr, sr, pc, sc, ncolg);
  } else {
    constexpr int NT = kRowColFosThreads, STR = kRowColFosStrips;
    ncolg = ceil_div(K, NT);
    if (mse)
      hipLaunchKernelGGL((k_rowcol<InT, true, true, NT, STR>), grid, block, 0, st, x, ga, D, M, K, pr, sr, pc, sc, ncolg);
    else
      hipLaunchKernelGGL((k_rowcol<InT, true, false, NT, STR>), grid, block, 0, st, x, ga, D, M, K, pr, sr, pc, sc, ncolg);
  }
  return (int)hipGetLastError();
}

int launch_rowcol(const void* x, int in_bf16, int64_t M, int64_t K, const float* global_amax,
                  int four_over_six, int mse, float bound, uint8_t* packed_row,
                  uint8_t* scales_row, uint8_t* packed_col, uint8_t* scales_col, void* stream) {
  if (M == 0 || K == 0) return 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float D = 6.0f * bound;
  if (in_bf16)
    return launch_rowcol_t(reinterpret_cast<const uint16_t*>(x), global_amax, four_over_six, mse, D,
                           M, K, packed_row, scales_row, packed_col, scales_col, st);
  return launch_rowcol_t(reinterpret_cast<const float*>(x), global_amax, four_over_six, mse, D, M, K,
                         packed_row, scales_row, packed_col, scales_col, st);
}

template <typename InT, bool MSE>
static int launch_4over6_2d_t(const InT* x, const float* ga, float D, int64_t M, int64_t K,
                              uint8_t* pr, uint8_t* pc, uint8_t* ts, hipStream_t st) {
  constexpr int NT = k46TileThreads, STR = k46TileStrips;
  const int64_t ncolg = ceil_div(K, NT);
  const int col = pc != nullptr;
  const int str = tile_strips_4over6_2d(M, K, col);  // STR whenever col
  const LaunchPlan pl = plan_4over6_2d(M, K, col);
  const dim3 grid((unsigned)pl.grid), block(pl.block);
  if (col) hipLaunchKernelGGL((k_4over6_2d<InT, MSE, true, NT, STR>), grid, block, 0, st, x, ga, D, M, K, pr, pc, ts, ncolg, str);
  else hipLaunchKernelGGL((k_4over6_2d<InT, MSE, false, NT, STR>), grid, block, 0, st, x, ga, D, M, K, pr, pc, ts, ncolg, str);
  return (int)hipGetLastError();
}

int launch_4over6_2d(const void* x, int in_bf16, int64_t M, int64_t K, const float* global_amax,
                     int mse, float bound, uint8_t* packed_row, uint8_t* packed_col,
                     uint8_t* tile_scales, void* stream) {
  if (M == 0 || K == 0) return 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float D = 6.0f * bound;
  if (in_bf16) {
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    return mse ? launch_4over6_2d_t<uint16_t, true>(xb, global_amax, D, M, K, packed_row, packed_col, tile_scales, st)
               : launch_4over6_2d_t<uint16_t, false>(xb, global_amax, D, M, K, packed_row, packed_col, tile_scales, st);
  }
  const float* xf = reinterpret_cast<const float*>(x);
  return mse ? launch_4over6_2d_t<float, true>(xf, global_amax, D, M, K, packed_row, packed_col, tile_scales, st)
             : launch_4over6_2d_t<float, false>(xf, global_amax, D, M, K, packed_row, packed_col, tile_scales, st);
}

}  // namespace nvfp4
