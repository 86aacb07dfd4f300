// OCP E4M3 encoding of K/V values, shared by every kernel that writes FP8
// codes into the pool (the pool-update kernel and the fused append of the
// verification launch), so that codes and scales are the same bit for bit
// whichever path writes them.
//
// Per-page scales (atozofsoftwareengineering.blog, section "Custom FP8
// Quantized Memory Block Layout", per-block scales S_K, S_V): a page-head
// written for the first time gets s = amax / 448 of the values written into
// it by that call (1 when amax is 0); a later append whose values exceed
// 448 s doubles s until they fit and re-encodes the page's codes.  Codes:
// y = x * (1/s) in fp32, clamped to +-448, rounded to nearest even.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

__device__ inline unsigned char quant_e4m3(float x, float inv) {
  float y = x * inv;
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  // hardware OCP E4M3 conversion, round to nearest even
  unsigned packed = __builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false);
  return static_cast<unsigned char>(packed & 0xFF);
}

// Scale of a page-head written for the first time, from the largest
// magnitude of the values written into it.
__device__ inline float fresh_page_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

// Scale of a page-head written before, for newly appended values whose
// largest magnitude is amax: unchanged when amax <= 448 s, else s doubled
// until it is (fp32 products and comparisons).  Codes already in the page
// are then encoded again (reencode_e4m3), a power-of-two change of scale.
__device__ inline float grown_page_scale(float amax, float s) {
  for (int i = 0; i < 256 && amax > 448.0f * s; ++i) s *= 2.0f;
  return s;
}

// A code of a page whose scale grows from s_old to s_new: the value it
// stands for, decode(c) * s_old in fp32, encoded with s_new.
__device__ inline unsigned char reencode_e4m3(unsigned char code, float s_old, float inv_new);

// E8M0 exponent byte of the tile scale 2^k for a tile whose largest magnitude
// is amax: k the smallest integer with amax / 2^k <= 448 = 0.875 * 2^9
// (amax = m * 2^E with m in [0.5, 1): k = E - 9, plus 1 when m > 0.875),
// clamped to [-127, 127]; k = 0 for amax = 0.
__device__ inline int tile_exponent_byte(float amax) {
  const unsigned b = __float_as_uint(amax);
  if (amax == 0.0f) return 127;
  const int e = int(b >> 23) & 0xFF;
  if (e == 0) return 0;                          // subnormal amax: k = -127
  const int k = (e - 126) - 9 + ((b & 0x7FFFFF) > 0x600000u ? 1 : 0);
  return min(max(k, -127), 127) + 127;
}

// Value of an E4M3 code (finite codes only; NaN codes are never written).
__device__ inline float dequant_e4m3(unsigned char code) {
  const unsigned s = code >> 7, e = (code >> 3) & 15u, m = code & 7u;
  const float mag = e ? ldexpf(float(8 + m), int(e) - 10) : ldexpf(float(m), -9);
  return s ? -mag : mag;
}

__device__ inline unsigned char reencode_e4m3(unsigned char code, float s_old, float inv_new) {
  return quant_e4m3(dequant_e4m3(code) * s_old, inv_new);
}

}  // namespace pkv
