// Helpers of the row-contiguous strip mapping of the 2D quantize kernel: in a
// strip of 16 rows, wave w of a 512-lane workgroup owns rows 2w and 2w + 1,
// and lane l holds columns 8l .. 8l + 7 of both rows, so a 16x16 tile is the
// lane pair (2t, 2t + 1) of all eight waves.
#pragma once

#include "nvfp4_device.hpp"

namespace nvfp4 {

constexpr int kStripLanes = 512;                // lanes (and columns) of a workgroup
constexpr int kStripTiles = kStripLanes / 16;   // tiles side by side (32)
constexpr int kStripWaves = kStripLanes / 64;   // waves; each owns 2 rows of a strip
constexpr int kStripCount = 16;                 // strips of 16 rows per workgroup

// Lane-pair partner's value (DPP quad permutation [1, 0, 3, 2]).
NV_DEV uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// Largest magnitude among N values as an fp32 bit pattern with NaNs dropped
// (0 for none), plus whether a NaN was seen.  Integer order of magnitude bit
// patterns is value order; patterns above 0x7F800000 are NaNs.
template <int N>
NV_DEV void absmax_nan_drop(const float* v, uint32_t& nd, uint32_t& fl) {
  uint32_t raw = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t m = f2bits(v[i]) & 0x7FFFFFFFu;
    raw = m > raw ? m : raw;
  }
  fl = 0u;
  nd = raw;
  if (raw > 0x7F800000u) {
    fl = 1u;
    nd = 0u;
    for (int i = 0; i < N; ++i) {
      const uint32_t m = f2bits(v[i]) & 0x7FFFFFFFu;
      if (m <= 0x7F800000u && m > nd) nd = m;
    }
  }
}

// NaN-dropping amax bits (fp32 pattern) and NaN flag of a lane's two rows of
// eight elements, from the raw loaded words.  bf16: the max of the 16-bit
// magnitude patterns of each half-word (one packed max per word); a pattern
// above 0x7F80 flags a NaN, then the slow NaN-dropping scan runs.
NV_DEV void lane_amax(const uint4* r, const uint16_t*, uint32_t& nd, uint32_t& fl) {
  const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 m = __builtin_bit_cast(us2, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[i] & 0x7FFF7FFFu));
  uint32_t h = m.x > m.y ? m.x : m.y;
  fl = 0u;
  if (h > 0x7F80u) {
    fl = 1u;
    h = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t e = (w[i >> 1] >> (16 * (i & 1))) & 0x7FFFu;
      if (e <= 0x7F80u && e > h) h = e;
    }
  }
  nd = h << 16;
}

NV_DEV void lane_amax(const uint4* r, const float*, uint32_t& nd, uint32_t& fl) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i] = bits2f(r[i].x);
    v[4 * i + 1] = bits2f(r[i].y);
    v[4 * i + 2] = bits2f(r[i].z);
    v[4 * i + 3] = bits2f(r[i].w);
  }
  absmax_nan_drop<16>(v, nd, fl);
}

// Eight values of one row: load (bf16 or fp32) and widen to fp32.
template <typename InT>
struct Row8 {
  static constexpr int kU4 = sizeof(InT) * 8 / 16;  // uint4 per 8 elements
};

NV_DEV void widen8(const uint4* r, const uint16_t*, float x[8]) {
  const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bits2f(w[i] << 16);
    x[2 * i + 1] = bits2f(w[i] & 0xFFFF0000u);
  }
}

NV_DEV void widen8(const uint4* r, const float*, float x[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    x[4 * i] = bits2f(r[i].x);
    x[4 * i + 1] = bits2f(r[i].y);
    x[4 * i + 2] = bits2f(r[i].z);
    x[4 * i + 3] = bits2f(r[i].w);
  }
}

// Rowwise codes of a tile's lane pair: ca holds the lane's eight codes of
// row A (= 2w), cb those of row B; the even lane stores 8 bytes of row A (its
// word, then its partner's), the odd lane 8 bytes of row B (its partner's
// word, then its own), so a wave store covers 256 contiguous bytes of both
// rows.  Both lanes of the pair must execute it; dst is the lane's 8-byte
// destination (row_dst_offset).
NV_DEV void store_rows_pair(uint8_t* dst, int lane, uint32_t ca, uint32_t cb) {
  const uint32_t oa = pair_swap(ca), ob = pair_swap(cb);
  *reinterpret_cast<uint2*>(dst) = (lane & 1) == 0 ? make_uint2(ca, oa) : make_uint2(ob, cb);
}

// Byte offset of a lane's rowwise store for the strip whose row A is rowA.
NV_DEV int64_t row_dst_offset(int64_t rowA, int64_t K, int64_t c0, int lane) {
  return (lane & 1) == 0 ? rowA * (K / 2) + c0 / 2 : (rowA + 1) * (K / 2) + (c0 - 8) / 2;
}

// Columnwise codes: a lane's two rows give one code byte for each of its
// eight columns (row A in the low nibble, row B in the high), byte wv of the
// column's 8-byte word of strip st.  The column's 16 words (128 bytes) sit in
// LDS at colbuf[column * 16 ..], word of strip st at (st + lane) & 15 (the
// rotation spreads a wave's byte writes over the banks).
NV_DEV void stage_col_bytes(uint2* colbuf, int lane, int wv, int st, uint32_t ca, uint32_t cb) {
  const uint32_t ev = (ca & 0x0F0F0F0Fu) | ((cb << 4) & 0xF0F0F0F0u);  // columns 0, 2, 4, 6
  const uint32_t od = ((ca >> 4) & 0x0F0F0F0Fu) | (cb & 0xF0F0F0F0u);  // columns 1, 3, 5, 7
  uint8_t* p = reinterpret_cast<uint8_t*>(colbuf) + (8 * lane) * (kStripCount * 8) +
               ((st + lane) & (kStripCount - 1)) * 8 + wv;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    p[(2 * k) * (kStripCount * 8)] = (uint8_t)(ev >> (8 * k));
    p[(2 * k + 1) * (kStripCount * 8)] = (uint8_t)(od >> (8 * k));
  }
}

// Write the column segments of a workgroup (after a barrier): 16 lanes per
// column, one 8-byte word (strip) each, so every store instruction covers
// four whole column segments of nst * 8 bytes.
NV_DEV void flush_col_segments(const uint2* colbuf, int64_t cg, int64_t sg, int nst, int64_t M,
                               int64_t K, uint8_t* packed_col) {
  const int q = threadIdx.x & 15;
  for (int cc = threadIdx.x >> 4; cc < kStripLanes; cc += kStripLanes / 16) {
    const int64_t col = cg * kStripLanes + cc;
    if (col < K && q < nst)
      *reinterpret_cast<uint2*>(packed_col + col * (M / 2) + sg * (kStripCount * 8) + q * 8) =
          colbuf[cc * kStripCount + ((q + (cc >> 3)) & (kStripCount - 1))];
  }
}

}  // namespace nvfp4
