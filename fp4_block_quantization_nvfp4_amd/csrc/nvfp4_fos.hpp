// Four-over-six building blocks shared by the 1x16 and the 16x16 kernels
// (four-over-six pull request "Add NVFP4 four-over-six (row-wise)
// quantization to the training prototype": What, numeric details, CuTe DSL
// kernel Design).
//
// A candidate (map-to-6 or map-to-4) is the block's codes under one e4m3
// scale s plus its dequantization error, summed in element order 0..15, of
// d = ((val * s) * A) / D against the input.  With A and D fixed, d depends
// only on the scale code and the code's magnitude, so kernels keep a table
// of d (and of the encode reciprocals rho) in LDS and look elements up.
#pragma once

#include "nvfp4_device.hpp"

namespace nvfp4 {

NV_DEV float e2m1_value(uint32_t m) {
  return m <= 4u ? (float)m * 0.5f : (m == 5u ? 3.0f : (m == 6u ? 4.0f : 6.0f));
}

constexpr int kDStride = 9;  // floats per scale code in the d table (8 used; 9 spreads LDS banks)
constexpr int kTabFloats = 128 + 127 * kDStride;  // rho[128] then d[127][kDStride]

// Fill rho[k] = min(1 / (s_k * S_dec), FLT_MAX) and d[k][m] = ((v_m * s_k) * A) / D
// for scale codes k in [kmin, kmax], shared by the nthreads lanes of the
// workgroup (lane `tid`).  The caller synchronizes afterwards.
NV_DEV void build_fos_tables(float* rhoT, float* dT, int kmin, int kmax, float A, float D,
                             float S_dec, int tid, int nthreads) {
  if (kmin > kmax) return;
  const float rD = 1.0f / D;
  for (int k = kmin + tid; k <= kmax; k += nthreads)
    rhoT[k] = encode_reciprocal(e4m3_decode((uint32_t)k), S_dec);
  const int n = (kmax - kmin + 1) * 8;
  for (int e = tid; e < n; e += nthreads) {
    const uint32_t k = (uint32_t)kmin + (uint32_t)(e >> 3);
    dT[k * kDStride + (e & 7)] = div_guarded((e2m1_value((uint32_t)(e & 7)) * e4m3_decode(k)) * A, D, rD);
  }
}

// Error sums of both candidates over a block, each in element order: t6 / t4
// point at the candidates' rows of the d table, c6 / c4 hold their 16 codes;
// element i's d is entry (code & 7).  The codes are first spread to one byte
// per element (4 * (code & 7); even elements from the low nibbles, odd from
// the high nibbles) so that each LDS address is one add with a byte-select
// operand; the empty asm keeps the compiler from re-deriving per-element
// shifts.  All 32 lookups are issued before the sums so the LDS latency of
// one block overlaps.  |x - d| and (x - d)^2 are unchanged when both signs
// flip, so the error is taken on magnitudes.
template <bool MSE>
NV_DEV void error_sums(const float xv[16], const float* t6, const uint32_t c6[2], const float* t4,
                       const uint32_t c4[2], float& E6, float& E4) {
  const char* tb6 = reinterpret_cast<const char*>(t6);
  const char* tb4 = reinterpret_cast<const char*>(t4);
  float d6[16], d4[16];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t ev6 = (c6[w] << 2) & 0x1C1C1C1Cu, od6 = (c6[w] >> 2) & 0x1C1C1C1Cu;
    uint32_t ev4 = (c4[w] << 2) & 0x1C1C1C1Cu, od4 = (c4[w] >> 2) & 0x1C1C1C1Cu;
    asm("" : "+v"(ev6), "+v"(od6), "+v"(ev4), "+v"(od4));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      d6[8 * w + 2 * b] = *reinterpret_cast<const float*>(tb6 + ((ev6 >> (8 * b)) & 0xFFu));
      d6[8 * w + 2 * b + 1] = *reinterpret_cast<const float*>(tb6 + ((od6 >> (8 * b)) & 0xFFu));
      d4[8 * w + 2 * b] = *reinterpret_cast<const float*>(tb4 + ((ev4 >> (8 * b)) & 0xFFu));
      d4[8 * w + 2 * b + 1] = *reinterpret_cast<const float*>(tb4 + ((od4 >> (8 * b)) & 0xFFu));
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float u6 = fabsf(xv[i]) - d6[i], u4 = fabsf(xv[i]) - d4[i];
    const float e6 = MSE ? u6 * u6 : fabsf(u6), e4 = MSE ? u4 * u4 : fabsf(u4);
    E6 = (i == 0) ? e6 : E6 + e6;
    E4 = (i == 0) ? e4 : E4 + e4;
  }
}

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

}  // namespace nvfp4
