// Test support: exhaustive scans of the gfx950 conversions the kernels use
// for the element codes (round-to-nearest and stochastic fp32 -> e2m1), the
// block scale bytes (fp32 -> e4m3 after the 448 cap) and the decodes
// (e2m1 -> fp32, e4m3 -> fp32).  Each scan calls the very device helpers of
// nvfp4_device.hpp, with the same operand placement as the kernels.
//
// The input of a scan is a run of 32-bit patterns p (as fp32 values, or code
// bytes for the decodes).  The run is cut into chunks of 2^L consecutive
// patterns, one lane per chunk; each lane computes y(p) for every pattern of
// its chunk and writes one record {y(first), y(last), number of p in the
// chunk with y(p) != y(p - 1), first such p}.  A host test compares those
// records with the oracle: equal values at every chunk end, and change points
// exactly where the oracle's (monotone) encoder changes, cover every pattern
// of the run without copying 2^32 results.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

constexpr uint32_t kOldWord = 0xA5A5A5A5u;  // bytes the e2m1 conversion must leave alone

template <int SEL>
NV_DEV uint32_t scan_rtn(float a, float b) {
  return hw_fp4_pair<SEL>(kOldWord, a, b);
}

template <int SEL>
NV_DEV uint32_t scan_sr(float a, float b, uint32_t nw) {
  return (hw_fp4_sr_pair<SEL>(a, b, nw) >> (8 * SEL)) & 0xFFu;
}

template <int SEL>
NV_DEV uint32_t scan_dec_fp4(uint32_t byte, bool hi) {
  const nv_f2 v = hw_fp4_values<SEL>(byte << (8 * SEL));
  return f2bits(hi ? v.y : v.x);
}

template <int SEL>
NV_DEV uint32_t scan_dec_e4m3(uint32_t code) {
  return f2bits(hw_e4m3_value<SEL>(code << (8 * SEL)));
}

// kind 0: round-to-nearest e2m1, param = SEL | slot << 2; the other element
//         is 0, the result is the whole word (old bytes 0xA5).
// kind 1: e4m3 scale byte of min(p, 448), param = slot (byte 0 or 1 of the
//         pair conversion, the other operand 0).
// kind 2: stochastic e2m1, param = u16 | SEL << 16 | slot << 18: the element
//         in `slot` takes the draw u16, the other element is 0 with draw
//         0x5A5A; the result is byte SEL.
// kind 3: e2m1 decode of byte p (p < 256), param = SEL | half << 2.
// kind 4: e4m3 decode of code p (p < 256), param = SEL (0 or 1).
NV_DEV uint32_t scan_value(int kind, uint32_t param, uint32_t p) {
  const float f = bits2f(p);
  const uint32_t sel = param & 3u;
  if (kind == 0) {
    const bool slot_b = (param >> 2) & 1u;
    const float a = slot_b ? 0.0f : f, b = slot_b ? f : 0.0f;
    switch (sel) {
      case 0: return scan_rtn<0>(a, b);
      case 1: return scan_rtn<1>(a, b);
      case 2: return scan_rtn<2>(a, b);
      default: return scan_rtn<3>(a, b);
    }
  }
  if (kind == 1) {
    const float s = fminf(f, kE4m3Max);
    return (param & 1u) ? (hw_e4m3_pair(0.0f, s) >> 8) : (hw_e4m3_pair(s, 0.0f) & 0xFFu);
  }
  if (kind == 2) {
    const uint32_t u = param & 0xFFFFu, s2 = (param >> 16) & 3u;
    const bool slot_b = (param >> 18) & 1u;
    const float a = slot_b ? 0.0f : f, b = slot_b ? f : 0.0f;
    const uint32_t w = slot_b ? (0x5A5Au | (u << 16)) : (u | (0x5A5Au << 16));
    switch (s2) {
      case 0: return scan_sr<0>(a, b, ~w);
      case 1: return scan_sr<1>(a, b, ~w);
      case 2: return scan_sr<2>(a, b, ~w);
      default: return scan_sr<3>(a, b, ~w);
    }
  }
  if (kind == 3) {
    const bool hi = (param >> 2) & 1u;
    switch (sel) {
      case 0: return scan_dec_fp4<0>(p, hi);
      case 1: return scan_dec_fp4<1>(p, hi);
      case 2: return scan_dec_fp4<2>(p, hi);
      default: return scan_dec_fp4<3>(p, hi);
    }
  }
  return (sel & 1u) ? scan_dec_e4m3<1>(p) : scan_dec_e4m3<0>(p);
}

__global__ __launch_bounds__(256) void k_selftest_scan(int kind, uint32_t param, uint64_t first,
                                                       uint64_t count, int chunk_log2,
                                                       uint64_t nchunks, uint4* __restrict__ rec) {
  const uint64_t c = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (c >= nchunks) return;
  const uint64_t lo = c << chunk_log2;
  const uint64_t len = (count - lo) < (uint64_t(1) << chunk_log2) ? (count - lo) : (uint64_t(1) << chunk_log2);
  uint32_t p = (uint32_t)(first + lo);
  const uint32_t y0 = scan_value(kind, param, p);
  uint32_t prev = y0, nchg = 0, pos = 0;
  for (uint64_t i = 1; i < len; ++i) {
    ++p;
    const uint32_t y = scan_value(kind, param, p);
    if (y != prev) {
      if (nchg == 0) pos = p;
      ++nchg;
    }
    prev = y;
  }
  rec[c] = make_uint4(y0, prev, nchg, pos);
}

int launch_selftest_scan(int kind, uint32_t param, uint64_t first, uint64_t count, int chunk_log2,
                         uint32_t* records, void* stream) {
  const uint64_t nchunks = (count + (uint64_t(1) << chunk_log2) - 1) >> chunk_log2;
  const dim3 grid((unsigned)((nchunks + 255) / 256)), block(256);
  hipLaunchKernelGGL(k_selftest_scan, grid, block, 0, reinterpret_cast<hipStream_t>(stream), kind, param,
                     first, count, chunk_log2, nchunks, reinterpret_cast<uint4*>(records));
  return (int)hipGetLastError();
}

}  // namespace nvfp4
