// Exact quantisers of the cache formats (device code), shared by the pack
// kernels and the compressor's append.
//
// Sources: "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
// (mer.run) section 5 (s_g = E4M3(max|x|/6), x_i -> E2M1(x_i/s_g)) and
// section 2 (MXFP4 indexer keys); "DeepSeek-V4.1-Flash, 2. Architecture"
// section 2.4.4.  Every rounding decision is taken on the exact real value:
// quotients by an E4M3 scale are never formed -- |x| is compared with s
// times each E2M1 rounding threshold, products that are exact in float32
// (s has <= 4 significant bits, the thresholds <= 3) -- and divisions by 6
// or by powers of two are done in float64, where the quotient cannot cross
// a rounding boundary of the 4- or 8-bit target (a float32 dividend has 24
// bits).
#pragma once
#include "common.h"

namespace csa2 {

// float64 value -> E4M3 ("FN") code, round to nearest even, saturate at 448.
__device__ __forceinline__ uint32_t e4m3_from_f64(double v) {
  const uint32_t sign = signbit(v) ? 0x80u : 0u;
  const double a = fabs(v);
  if (a >= 448.0) return sign | 0x7Eu;
  if (a < 0.015625) {                    // below 2^-6: grid of 2^-9
    return sign | (uint32_t)rint(a * 512.0);   // 8 -> code 8 = 2^-6
  }
  const int e = ilogb(a);                // -6 .. 8
  const double m = rint((ldexp(a, -e) - 1.0) * 8.0);   // 0 .. 8
  uint32_t code = (uint32_t)((e + 7) * 8) + (uint32_t)m; // 8 carries up
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e == 0 ? (float)m * 0.001953125f
                     : ldexpf(1.0f + 0.125f * (float)m, (int)e - 7);
  if (e == 15 && m == 7) mag = __builtin_nanf("");
  return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  float mag = m < 2 ? 0.5f * (float)m
                    : ldexpf(1.0f + 0.5f * (float)(m & 1u), (int)(m >> 1) - 1);
  return (c & 8u) ? -mag : mag;
}

// E2M1 code of x / s for an E4M3 value s > 0, decided by exact float32
// comparisons of |x| with s times the rounding thresholds.  The tie at each
// threshold goes to the even code: strict '>' where the lower neighbour is
// even, '>=' where the upper one is.
__device__ __forceinline__ uint32_t e2m1_code_scaled(float x, float s) {
  const float a = fabsf(x);
  uint32_t c = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) +
               (a >= 1.75f * s) + (a > 2.5f * s) + (a >= 3.5f * s) +
               (a > 5.0f * s);
  return c | (signbit(x) ? 8u : 0u);
}

// E2M1 code of the exact real r (float64), same rule.
__device__ __forceinline__ uint32_t e2m1_code_f64(double r) {
  const double a = fabs(r);
  uint32_t c = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) +
               (a > 2.5) + (a >= 3.5) + (a > 5.0);
  return c | (signbit(r) ? 8u : 0u);
}

// float64 value -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t bf16_from_f64(double v) {
  const uint32_t sign = signbit(v) ? 0x8000u : 0u;
  const double a = fabs(v);
  if (a == 0.0) return (uint16_t)sign;
  int e = ilogb(a);
  if (e < -126) e = -126;
  const double r = ldexp(rint(ldexp(a, 7 - e)), e - 7);   // 8 significant bits
  const float f = (float)r;                                // exact or +inf
  return (uint16_t)((f2u(f) >> 16) | sign);
}


// One 16-channel group of a main row: scale code s_g = E4M3(amax / 6)
// and the 16 E2M1 codes (two per byte, low nibble first) as two words.
__device__ __forceinline__ void quant_main_group(const float (&x)[16],
                                                 uint32_t (&w)[2],
                                                 uint32_t& sc) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  sc = e4m3_from_f64((double)amax / 6.0);
  const float s = e4m3_to_f32(sc);
  w[0] = 0u;
  w[1] = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = s > 0.0f ? e2m1_code_scaled(x[i], s)
                                : (signbit(x[i]) ? 8u : 0u);
    w[i >> 3] |= c << (4 * (i & 7));
  }
}

// One 32-element OCP MX block: E8M0 scale byte (shared exponent
// floor(log2 amax) - 2, clamped) and 32 E2M1 codes as four words.
__device__ __forceinline__ void quant_idx_block(const float (&x)[32],
                                                uint32_t (&w)[4],
                                                uint32_t& scale_byte) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  int e = -127;
  if (amax > 0.0f) {
    e = ilogb((double)amax) - 2;           // largest E2M1 exponent is 2
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  const double inv = ldexp(1.0, -e);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e2m1_code_f64((double)x[i] * inv);
    w[i >> 3] |= c << (4 * (i & 7));
  }
  scale_byte = (uint32_t)(e + 127);
}

}  // namespace csa2
