// Four-over-six building blocks shared by the 1x16 and the 16x16 kernels
// (four-over-six pull request "Add NVFP4 four-over-six (row-wise)
// quantization to the training prototype": What, numeric details, CuTe DSL
// kernel Design).
//
// A candidate (map-to-6 or map-to-4) is the block's codes under one e4m3
// scale s plus its dequantization error, summed in element order 0..15, of
// d = ((val * s) * A) / D against the input.  Kernels keep the encode
// reciprocals rho of all 127 scale codes in LDS and decide between the
// candidates from error sums in the scaled domain whenever a rounding bound
// proves the decision (certified_pick below); otherwise they compute the
// exact error sums.
#pragma once

#include "nvfp4_device.hpp"

namespace nvfp4 {

// Codes of one candidate: v = x * rho, rounded to e2m1 by the hardware
// conversion, two elements per instruction, even element in the low nibble.
// Only for blocks with no NaN (a negative NaN would encode 0xF).
NV_DEV void encode16_hw(const float xv[16], float rho, uint32_t c[2]) {
  c[0] = hw_fp4_pair<0>(0u, xv[0] * rho, xv[1] * rho);
  c[0] = hw_fp4_pair<1>(c[0], xv[2] * rho, xv[3] * rho);
  c[0] = hw_fp4_pair<2>(c[0], xv[4] * rho, xv[5] * rho);
  c[0] = hw_fp4_pair<3>(c[0], xv[6] * rho, xv[7] * rho);
  c[1] = hw_fp4_pair<0>(0u, xv[8] * rho, xv[9] * rho);
  c[1] = hw_fp4_pair<1>(c[1], xv[10] * rho, xv[11] * rho);
  c[1] = hw_fp4_pair<2>(c[1], xv[12] * rho, xv[13] * rho);
  c[1] = hw_fp4_pair<3>(c[1], xv[14] * rho, xv[15] * rho);
}

// Software round-to-nearest codes of a block (any input, NaN included: a
// NaN v encodes +6, code 0x7).
NV_DEV void encode16_sw(const float xv[16], float rho, uint32_t c[2]) {
  c[0] = 0u;
  c[1] = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = fabsf(xv[i]) * rho;
    float q;
    const uint32_t mag = e2m1_rtn(v, q);
    const uint32_t neg = (v != v) ? 0u : (f2bits(xv[i]) >> 31);
    const uint32_t code = mag | (neg << 3);
    if (i < 8) c[0] |= code << (4 * i);
    else c[1] |= code << (4 * (i - 8));
  }
}

// One candidate on the table-free path: codes and the element-order error
// sum with a true division per element.
template <bool MSE>
NV_DEV float candidate(const float xv[16], float s, float rho, float A, float D, uint32_t& c0,
                       uint32_t& c1) {
  float E = 0.0f;
  c0 = 0;
  c1 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float ax = fabsf(xv[i]);
    const float v = ax * rho;
    float q;
    const uint32_t mag = e2m1_rtn(v, q);
    const uint32_t neg = (v != v) ? 0u : (f2bits(xv[i]) >> 31);
    const uint32_t code = mag | (neg << 3);
    if (i < 8) c0 |= code << (4 * i);
    else c1 |= code << (4 * (i - 8));
    const float d = ((q * s) * A) / D;
    const float t = ax - d;
    const float e = MSE ? t * t : fabsf(t);
    E = (i == 0) ? e : E + e;
  }
  return E;
}

// ---------------------------------------------------------------------------
// Certified candidate choice without the per-element dequant values.
//
// The exact rule compares E_c = sum_i e_i (in element order, e_i = |x_i - d_i|
// or (x_i - d_i)^2, d_i = fl(fl(q_i s_c A) / D)) for c = 4 and 6.  Both
// candidates' codes come from v_i = fl(|x_i| rho_c), rho_c = fl(1 / W_c),
// W_c = fl(s_c S_dec), S_dec = fl(A / D), so the kernel already holds v_i
// and (by the exact hardware fp4 -> fp32 conversion) q_i.  Let c = s_c A / D
// (real), S = sum |x_i| <= N a (N elements, amax a), T = sum ||x_i| - q_i c|,
// u = 2^-24.  Every d_i carries two roundings (|d_i - q_i c| <= 2.01 u q_i c,
// and c sum q_i <= S + T), every e_i one more, and the element-order sum
// 15 u sum e_i (19 u for 16 row sums combined by a depth-4 tree), so
//   |E_c - T| <= 2.02 u S + 18.1 u T            (1x16; 22.1 u T for tiles).
// On the approximate side v_i = (|x_i| / c)(1 + eta_i), |eta_i| <= 4.01 u (S_dec,
// W, rho and the product), and Z_c = fl(W_c E'_c) with E'_c = sum |v_i - q_i|:
//   |Z_c - T| <= 4.02 u S + 19.1 u T            (1x16; 23.1 u T for tiles).
// Hence |Z_c - E_c| <= 6.04 u S + 37.2 u T (45.2 u T), and with S <= 16 a
// (256 a) both candidates together stay below 194 u a + 38 u (Z_4 + Z_6)
// (3092 u a + 46 u (Z_4 + Z_6) for tiles).  The margin B = k a + 2^-15 (Z_4
// + Z_6) + 2^-90, k = 2^-15 for 1x16 and 2^-11 for tiles, covers these at
// least 2.6 times over (the 2^-90 term covers subnormal products).
// For MSE (E'_c = sum (v_i - q_i)^2, Z_c = W_c^2 E'_c) let T_i = |x_i| - q_i c
// and E* = sum T_i^2.  Here v_i - q_i is exact (Sterbenz: v_i <= 12 in the
// guards), W_c (v_i - q_i) = (1 + g) T_i + |x_i| xi_i with |g| <= 2.01 u,
// |xi_i| <= 4.02 u, and |x_i - d_i| = T_i - q_i c beta_i, |beta_i| <= 2.01 u,
// so both sides carry cross terms sum |T_i| |x_i| <= 4 a sqrt(E*)
// (Cauchy-Schwarz over 16 elements of magnitude <= a):
//   |E_c - E*| <= 22.2 u E* + 16.2 u a sqrt(E*) + 132 u^2 a^2,
//   |Z_c - E*| <= 22.1 u E* + 32.3 u a sqrt(E*) + 260 u^2 a^2.
// The second gives sqrt(E*) <= (1 + 22.2 u) sqrt(Z_c) + 48.6 u a, hence
// |Z_c - E_c| <= 44.4 u Z_c + 48.6 u a sqrt(Z_c) + 2750 u^2 a^2, and for both
// candidates (sqrt(Z_4) + sqrt(Z_6) <= sqrt(2 (Z_4 + Z_6))) at most
// 44.4 u (Z_4 + Z_6) + 68.8 u a sqrt(Z_4 + Z_6) + 5500 u^2 a^2.  A 1x16 MSE
// margin B = 2^-16 a sqrt(Z_4 + Z_6) + 2^-30 a^2 + 2^-15 (Z_4 + Z_6) + 2^-90
// covers these 3.7, 48 and 11.5 times over (the square root is the hardware
// one, within an ulp; a scale code rounds sigma up by at most 2x, so
// W_c <= (a / 2)(1 + 6 u) and the a^2 term also covers the absolute error of
// a subnormal v_i).  Tiles keep the coarser bound with
// |x_i| |t_i| <= (x_i^2 + t_i^2) / 2: 3084 u a^2 + 59 u (Z_4 + Z_6), margin
// 2^-11 a^2 + 2^-15 (Z_4 + Z_6) + 2^-90.  Then
//   Z_4 + B < Z_6  proves E_4 < E_6 (map-to-4), and
//   Z_4 - B >= Z_6 proves E_4 >= E_6 (map-to-6, ties included).
// The range guards (2^-50 <= W_6 <= W_4 <= 2^50, a <= 2^50, finite Z, no
// NaN) keep every d_i, v_i and partial sum normal and finite.  Undecided
// blocks (exact ties occur in real data) take exact_error16 below; blocks
// outside the guards (NaN, infinities, zero or clipped scales) take the
// software candidate.

// Approximate error sum of one candidate from its scaled values v (signed,
// x * rho) and its codes c (q_i has the sign of v_i, so |v_i - q_i| is the
// distance of the magnitudes).
template <bool MSE>
NV_DEV float approx_error16(const float v[16], const uint32_t c[2]) {
  float q[16];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const nv_f2 p0 = hw_fp4_values<0>(c[w]), p1 = hw_fp4_values<1>(c[w]);
    const nv_f2 p2 = hw_fp4_values<2>(c[w]), p3 = hw_fp4_values<3>(c[w]);
    q[8 * w + 0] = p0.x; q[8 * w + 1] = p0.y; q[8 * w + 2] = p1.x; q[8 * w + 3] = p1.y;
    q[8 * w + 4] = p2.x; q[8 * w + 5] = p2.y; q[8 * w + 6] = p3.x; q[8 * w + 7] = p3.y;
  }
  float E = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float t = v[i] - q[i];
    E = MSE ? __builtin_fmaf(t, t, E) : E + fabsf(t);
  }
  return E;
}

// 1 / D computed where it is written: the empty asm statement hides D's
// value, so the division is not hoisted out of the rare exact path into the
// prologue of every wave.
NV_DEV float recip_in_place(float D) {
  asm volatile("" : "+v"(D));
  return 1.0f / D;
}

// Exact element-order error sum of one candidate with codes c (finite
// inputs, scale s, inside the range guards).  A code value is q = mu 2^k
// with mu in {1, 1.5}, so fl(q s A) = 2^k fl(mu s A) and
// d = fl(fl(q s A) / D) = 2^k fl(fl(mu s A) / D) while everything stays
// normal: two correctly rounded divisions per candidate instead of one per
// element.  2^k is q's exponent field (0 for q = 0), mu is its top mantissa
// bit.
// rD = 1 / D (see recip_in_place).
template <bool MSE>
NV_DEV float exact_error16(const float xv[16], const uint32_t c[2], float s, float A, float D,
                           float rD) {
  const float Q1 = div_guarded(s * A, D, rD);
  const float Q15 = div_guarded((1.5f * s) * A, D, rD);
  float E = 0.0f;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      nv_f2 p;
      if (b == 0) p = hw_fp4_values<0>(c[w]);
      else if (b == 1) p = hw_fp4_values<1>(c[w]);
      else if (b == 2) p = hw_fp4_values<2>(c[w]);
      else p = hw_fp4_values<3>(c[w]);
      const float qv[2] = {p.x, p.y};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 8 * w + 2 * b + h;
        const uint32_t qb = f2bits(qv[h]);
        const float d = bits2f(qb & 0x7F800000u) * ((qb & 0x400000u) ? Q15 : Q1);
        const float t = fabsf(xv[i]) - d;
        const float e = MSE ? t * t : fabsf(t);
        E = (i == 0) ? e : E + e;
      }
    }
  }
  return E;
}

// Exact tie without the exact sums.  When s4 = 1.5 s6 exactly and every
// map-to-6 value is exactly 1.5 times the map-to-4 value of the same element
// (zeros of either sign included), the products q s of the two candidates are
// equal as real numbers, so every later rounding of ((q s) A) / D, every
// error term and the element-order sums agree: E_4 = E_6, which keeps
// map-to-6.  Most exact ties of weight-like tensors are of this kind.
NV_DEV bool same_dequant16(const uint32_t c6[2], const uint32_t c4[2], float s6, float s4) {
  if (s4 != 1.5f * s6) return false;
  bool same = true;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    nv_f2 p6[4], p4[4];
    p6[0] = hw_fp4_values<0>(c6[w]); p4[0] = hw_fp4_values<0>(c4[w]);
    p6[1] = hw_fp4_values<1>(c6[w]); p4[1] = hw_fp4_values<1>(c4[w]);
    p6[2] = hw_fp4_values<2>(c6[w]); p4[2] = hw_fp4_values<2>(c4[w]);
    p6[3] = hw_fp4_values<3>(c6[w]); p4[3] = hw_fp4_values<3>(c4[w]);
#pragma unroll
    for (int b = 0; b < 4; ++b) same = same && p6[b].x == 1.5f * p4[b].x && p6[b].y == 1.5f * p4[b].y;
  }
  return same;
}

// 1: map-to-4 proven, 0: map-to-6 proven, -1: undecided inside the range
// guards (use exact_error16), -2: outside them (use the software
// candidate).  kLog2N = 4 for a 1x16 block, 8 for a 16x16 tile (E6a / E4a
// then the tile totals).
// The 1x16 MSE margin of the comment above: 2^-16 a sqrt(Zs) + 2^-30 a^2 +
// 2^-15 Zs + 2^-90 with Zs = Z4 + Z6 (finite and at most 2^111 inside the
// range guards).
NV_DEV float mse_margin16(float a, float Zs) {
  return __builtin_fmaf(a, __builtin_fmaf(__builtin_amdgcn_sqrtf(Zs), 0x1p-16f, a * 0x1p-30f),
                        __builtin_fmaf(Zs, 0x1p-15f, 0x1p-90f));
}

template <bool MSE, int kLog2N>
NV_DEV int certified_pick(float E6a, float E4a, float W6, float W4, float a) {
  if (!(W6 >= 0x1p-50f && W4 <= 0x1p50f && a <= 0x1p50f)) return -2;
  if (E6a != E6a || E4a != E4a) return -2;  // a NaN in the block
  const float Z6 = MSE ? (W6 * W6) * E6a : W6 * E6a;
  const float Z4 = MSE ? (W4 * W4) * E4a : W4 * E4a;
  if (!(Z6 <= kFltMax && Z4 <= kFltMax)) return -2;
  constexpr float kA = kLog2N == 4 ? 0x1p-15f : 0x1p-11f;
  const float B = (MSE && kLog2N == 4) ? mse_margin16(a, Z4 + Z6)
                                       : kA * (MSE ? a * a : a) + 0x1p-15f * (Z4 + Z6) + 0x1p-90f;
  if (Z4 + B < Z6) return 1;
  if (Z4 - B >= Z6) return 0;
  return -1;
}

// One candidate's codes (hardware encode, finite input) and approximate
// error sum, pair by pair: scale two elements, encode them into byte SEL,
// convert the byte back (exact) and accumulate |v - q| (or (v - q)^2), so
// no per-element array stays live.
template <bool MSE, int SEL>
NV_DEV void fos_pair(float x0, float x1, float rho, uint32_t& c, float& E) {
  const float v0 = x0 * rho, v1 = x1 * rho;
  c = hw_fp4_pair<SEL>(c, v0, v1);
  const nv_f2 q = hw_fp4_values<SEL>(c);
  const float t0 = v0 - q.x, t1 = v1 - q.y;
  if (MSE) {
    E = __builtin_fmaf(t0, t0, E);
    E = __builtin_fmaf(t1, t1, E);
  } else {
    E = E + fabsf(t0);
    E = E + fabsf(t1);
  }
}

template <bool MSE>
NV_DEV void fos_candidate(const float xv[16], float rho, uint32_t c[2], float& E) {
  // the four conversions of each word write all four of its bytes
  c[0] = any_u32();
  c[1] = any_u32();
  E = 0.0f;
  fos_pair<MSE, 0>(xv[0], xv[1], rho, c[0], E);
  fos_pair<MSE, 1>(xv[2], xv[3], rho, c[0], E);
  fos_pair<MSE, 2>(xv[4], xv[5], rho, c[0], E);
  fos_pair<MSE, 3>(xv[6], xv[7], rho, c[0], E);
  fos_pair<MSE, 0>(xv[8], xv[9], rho, c[1], E);
  fos_pair<MSE, 1>(xv[10], xv[11], rho, c[1], E);
  fos_pair<MSE, 2>(xv[12], xv[13], rho, c[1], E);
  fos_pair<MSE, 3>(xv[14], xv[15], rho, c[1], E);
}

// Both candidates of a block: codes and approximate error sums E'_6, E'_4.
template <bool MSE>
NV_DEV void fos_candidates(const float xv[16], float rho6, float rho4, uint32_t c6[2],
                           uint32_t c4[2], float& E6a, float& E4a) {
  fos_candidate<MSE>(xv, rho6, c6, E6a);
  fos_candidate<MSE>(xv, rho4, c4, E4a);
}

// Scale codes of both candidates: byte 0 map-to-6, byte 1 map-to-4 (each
// sigma capped at 448 first; hardware round-to-nearest-even e4m3).  The
// 7-bit masks only matter for a negative amax, which is invalid input: they
// keep table indexes in range.
NV_DEV uint32_t fos_scale_codes(float sig6) {
  return hw_e4m3_pair(fminf(sig6, kE4m3Max), fminf(sig6 * 1.5f, kE4m3Max)) & 0x7F7Fu;
}

// Four-over-six for one 1x16 block of a row or tensor with amax A: scale
// codes, both candidates by the hardware encode, then the certified choice,
// the exact sums of exact_error16 for undecided blocks, or the software
// candidate (software encoder, true divisions) outside the range guards.  a
// is the block's NaN-dropping amax, rhoT the encode reciprocals of all 127
// scale codes for S_dec.  Returns the scale byte.
template <bool MSE>
NV_DEV uint32_t fos_block(const float xv[16], float a, float S_enc, float S_dec, float A, float D,
                          const float* rhoT, uint32_t c[2]) {
  const uint32_t kk = fos_scale_codes(div_guarded(a, 6.0f, 1.0f / 6.0f) * S_enc);
  const uint32_t k6 = kk & 0xFFu, k4 = kk >> 8;
  const float rho6 = rhoT[k6], rho4 = rhoT[k4];
  const float s6 = hw_e4m3_value<0>(kk), s4 = hw_e4m3_value<1>(kk);
  uint32_t c6[2], c4[2];
  float E6a, E4a;
  fos_candidates<MSE>(xv, rho6, rho4, c6, c4, E6a, E4a);
  int pick = certified_pick<MSE, 4>(E6a, E4a, s6 * S_dec, s4 * S_dec, a);
  if (pick == -1) {
    if (same_dequant16(c6, c4, s6, s4)) {
      pick = 0;
    } else {
      const float rD = recip_in_place(D);
      const float E6 = exact_error16<MSE>(xv, c6, s6, A, D, rD);
      const float E4 = exact_error16<MSE>(xv, c4, s4, A, D, rD);
      pick = E4 < E6 ? 1 : 0;
    }
  } else if (pick == -2) {
    const float E6 = candidate<MSE>(xv, s6, rho6, A, D, c6[0], c6[1]);
    const float E4 = candidate<MSE>(xv, s4, rho4, A, D, c4[0], c4[1]);
    pick = E4 < E6 ? 1 : 0;
  }
  c[0] = pick ? c4[0] : c6[0];
  c[1] = pick ? c4[1] : c6[1];
  return pick ? k4 : k6;
}

// The same without the range guards, for a "plain" block: it holds no NaN,
// its amax a is finite with 2^-117 <= a <= A (a / 6 by the fast exact
// division, and sigma6 <= bound), its map-to-6 scale is not zero, and its
// tensor or row passed fos_row_in_range.  Then 2^-50 <= W6 <= W4 <= 2^50, a <= 2^50 and
// every v_i <= 12, so every Z is finite and no guard of certified_pick is
// needed.  Other blocks take the general fos_block.  With TIES, undecided
// blocks first try same_dequant16.
NV_DEV bool fos_row_in_range(float A, float S_dec) {
  return A <= 0x1p50f && S_dec >= 0x1p-41f && S_dec <= 0x1p41f;
}

// With WTAB, WT holds W = s * S_dec for every scale code (the same product
// the block would form), tabulated per row beside rhoT.  The MAE margin is
// formed as fma(a + (Z4 + Z6), 2^-15, 2^-90), the MSE one by mse_margin16,
// and the test compares fl(Z6 - Z4) with +-B: the same bounds as in
// certified_pick up to a few roundings of relative size 2^-24, far inside
// their safety factors (fl(Z6 - Z4) > B implies Z6 - Z4 > B / (1 + 2^-24)).
template <bool MSE, bool TIES, bool WTAB = false>
NV_DEV uint32_t fos_block_plain(const float xv[16], float a, bool plain, float S_enc, float S_dec,
                                float A, float D, const float* rhoT, uint32_t c[2],
                                const float* WT = nullptr) {
  const uint32_t kk = fos_scale_codes(div_fast(a, 6.0f, 1.0f / 6.0f) * S_enc);
  const uint32_t k6 = kk & 0xFFu, k4 = kk >> 8;
  if (!plain || k6 == 0u) return fos_block<MSE>(xv, a, S_enc, S_dec, A, D, rhoT, c);
  const float rho6 = rhoT[k6], rho4 = rhoT[k4];
  uint32_t c6[2], c4[2];
  float E6a, E4a;
  fos_candidates<MSE>(xv, rho6, rho4, c6, c4, E6a, E4a);
  const float W6 = WTAB ? WT[k6] : hw_e4m3_value<0>(kk) * S_dec;
  const float W4 = WTAB ? WT[k4] : hw_e4m3_value<1>(kk) * S_dec;
  const float Z6 = (MSE ? W6 * W6 : W6) * E6a;
  const float Z4 = (MSE ? W4 * W4 : W4) * E4a;
  const float B = MSE ? mse_margin16(a, Z4 + Z6) : __builtin_fmaf(a + (Z4 + Z6), 0x1p-15f, 0x1p-90f);
  const float dZ = Z6 - Z4;
  int pick;
  if (dZ > B) {
    pick = 1;
  } else if (dZ <= -B) {
    pick = 0;
  } else if (TIES && same_dequant16(c6, c4, hw_e4m3_value<0>(kk), hw_e4m3_value<1>(kk))) {
    pick = 0;
  } else {
    const float s6 = hw_e4m3_value<0>(kk), s4 = hw_e4m3_value<1>(kk);
    const float rD = recip_in_place(D);
    const float E6 = exact_error16<MSE>(xv, c6, s6, A, D, rD);
    const float E4 = exact_error16<MSE>(xv, c4, s4, A, D, rD);
    pick = E4 < E6 ? 1 : 0;
  }
  c[0] = pick ? c4[0] : c6[0];
  c[1] = pick ? c4[1] : c6[1];
  return pick ? k4 : k6;
}

// A block of 16 fp32 values with the tensor's (or row's) amax A and `lean` =
// fos_row_in_range(A, S_dec): the largest magnitude bit pattern tells finite
// blocks from blocks with a NaN or an infinity (those take fos_block with the
// NaN-dropping amax); a finite block is plain when 2^-117 <= a <= A.
// The same with the block's largest magnitude bit pattern ab given (integer
// max of the |x| patterns: a NaN pattern tops it, so ab >= 0x7F800000 flags a
// NaN or an infinity).
template <bool MSE, bool TIES, bool WTAB = false>
NV_DEV uint32_t fos_block_ab(const float xv[16], uint32_t ab, bool lean, float S_enc, float S_dec,
                             float A, float D, const float* rhoT, uint32_t c[2],
                             const float* WT = nullptr) {
  if (ab < 0x7F800000u) {
    const float a = bits2f(ab);
    return fos_block_plain<MSE, TIES, WTAB>(xv, a, lean && a >= 0x1p-117f && a <= A, S_enc, S_dec, A,
                                            D, rhoT, c, WT);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, abs_nan0(xv[i]));
  return fos_block<MSE>(xv, a, S_enc, S_dec, A, D, rhoT, c);
}

template <bool MSE, bool TIES, bool WTAB = false>
NV_DEV uint32_t fos_block_f32(const float xv[16], bool lean, float S_enc, float S_dec, float A,
                              float D, const float* rhoT, uint32_t c[2], const float* WT = nullptr) {
  uint32_t ab = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t m = f2bits(xv[i]) & 0x7FFFFFFFu;
    ab = m > ab ? m : ab;
  }
  return fos_block_ab<MSE, TIES, WTAB>(xv, ab, lean, S_enc, S_dec, A, D, rhoT, c, WT);
}

}  // namespace nvfp4
