// Cache write path: FP4 main-KV, MXFP4 indexer-key and E4M3 window packing,
// exact dequantisation, and pooled bf16 block keys.
//
// Sources: "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
// (mer.run) section 5, quantiser equation s_g = E4M3(max|x|/6),
// x_i -> E2M1(x_i/s_g), and section 2 (288 B / 68 B entries);
// "DeepSeek-V4.1-Flash, 2. Architecture" section 2.4.4 (E2M1 + one E4M3
// scale per 16 channels, no global scale; MXFP4 indexer keys; FP8 window).
//
// Every rounding decision is taken on the exact real value: quotients by an
// E4M3 scale are never formed -- |x| is compared with s times each E2M1
// rounding threshold, products that are exact in float32 (s has <= 4
// significant bits, the thresholds <= 3) -- and divisions by 6 or by powers
// of two are done in float64, where the quotient cannot cross a rounding
// boundary of the 4- or 8-bit target (a float32 dividend has 24 bits).
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

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

// One thread per 16-channel group of a main row.
__global__ void pack_main_kernel(const float* __restrict__ src, int64_t n,
                                 uint8_t* __restrict__ codes,
                                 uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * 32) return;
  const int64_t row = t >> 5;
  const int g = (int)(t & 31);
  const float4* p = reinterpret_cast<const float4*>(src + row * 512 + g * 16);
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = p[i];
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const uint32_t sc = e4m3_from_f64((double)amax / 6.0);
  const float s = e4m3_to_f32(sc);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = s > 0.0f ? e2m1_code_scaled(x[i], s)
                                : (signbit(x[i]) ? 8u : 0u);
    w[i >> 3] |= c << (4 * (i & 7));
  }
  *reinterpret_cast<uint2*>(codes + row * 256 + g * 8) = make_uint2(w[0], w[1]);
  scales[row * 32 + g] = (uint8_t)sc;
}

// One thread per 32-element MX block of an indexer row.
__global__ void pack_idx_kernel(const float* __restrict__ src, int64_t n,
                                uint8_t* __restrict__ codes,
                                uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * 4) return;
  const int64_t row = t >> 2;
  const int blk = (int)(t & 3);
  const float4* p = reinterpret_cast<const float4*>(src + row * 128 + blk * 32);
  float x[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = p[i];
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  int e = -127;
  if (amax > 0.0f) {
    e = ilogb((double)amax) - 2;           // largest E2M1 exponent is 2
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  const double inv = ldexp(1.0, -e);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e2m1_code_f64((double)x[i] * inv);
    w[i >> 3] |= c << (4 * (i & 7));
  }
  *reinterpret_cast<uint4*>(codes + row * 64 + blk * 16) =
      make_uint4(w[0], w[1], w[2], w[3]);
  scales[row * 4 + blk] = (uint8_t)(e + 127);
}

// One thread per 4 window values.
__global__ void pack_swa_kernel(const float* __restrict__ src, int64_t n4,
                                uint32_t* __restrict__ codes) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(src)[t];
  codes[t] = e4m3_from_f64(v.x) | (e4m3_from_f64(v.y) << 8) |
             (e4m3_from_f64(v.z) << 16) | (e4m3_from_f64(v.w) << 24);
}

// One thread per code byte (two values).
__global__ void unpack_kernel(int fmt, const uint8_t* __restrict__ codes,
                              const uint8_t* __restrict__ scales, int64_t n,
                              float* __restrict__ dst) {
  const int bytes_per_row = fmt == 0 ? 256 : (fmt == 1 ? 64 : 512);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * bytes_per_row) return;
  const uint32_t b = codes[t];
  if (fmt == 2) {          // one E4M3 value per byte
    dst[t] = e4m3_to_f32(b);
    return;
  }
  const int64_t row = t / bytes_per_row;
  const int j = (int)(t % bytes_per_row);
  float lo = e2m1_to_f32(b & 15u), hi = e2m1_to_f32(b >> 4);
  if (fmt == 0) {
    const float s = e4m3_to_f32(scales[row * 32 + (j >> 3)]);
    lo *= s; hi *= s;
  } else {
    const int ex = (int)scales[row * 4 + (j >> 4)] - 127;
    lo = ldexpf(lo, ex); hi = ldexpf(hi, ex);
  }
  reinterpret_cast<float2*>(dst)[t] = make_float2(lo, hi);
}

// One thread per (sequence, block, dim).
__global__ void block_keys_kernel(const uint8_t* __restrict__ codes,
                                  const uint8_t* __restrict__ scales,
                                  int64_t n_cap, const int32_t* __restrict__ n_entries,
                                  int64_t nb, int block,
                                  uint16_t* __restrict__ keys, int64_t total) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int d = (int)(t & 127);
  const int64_t jb = (t >> 7) % nb;
  const int64_t b = (t >> 7) / nb;
  int64_t n = n_entries[b];
  n = n < 0 ? 0 : (n > n_cap ? n_cap : n);        // never past the cache
  const int64_t start = jb * block;
  uint16_t out = 0;
  if (start < n) {
    const int64_t cnt = (n - start) < block ? (n - start) : block;
    double sum = 0.0;
    for (int64_t r = 0; r < cnt; ++r) {
      const int64_t row = b * n_cap + start + r;
      const uint32_t byte = codes[row * 64 + (d >> 1)];
      const uint32_t c = (d & 1) ? (byte >> 4) : (byte & 15u);
      sum += ldexp((double)e2m1_to_f32(c), (int)scales[row * 4 + (d >> 5)] - 127);
    }
    out = bf16_from_f64(sum / (double)cnt);
  }
  keys[t] = out;
}

// Visible blocks per sequence: ceil(n_entries / block).
__global__ void nblocks_kernel(const int32_t* __restrict__ n_entries, int B,
                               int block, int32_t* __restrict__ nblk) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t n = n_entries[b] > 0 ? n_entries[b] : 0;
  nblk[b] = (n + block - 1) / block;
}

inline unsigned grid_for(int64_t n, int threads) {
  return (unsigned)((n + threads - 1) / threads);
}

}  // namespace

hipError_t launch_pack_main(const float* src, int64_t n, uint8_t* codes,
                            uint8_t* scales, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_main_kernel, dim3(grid_for(n * 32, 256)), dim3(256),
                     0, s, src, n, codes, scales);
  return hipGetLastError();
}

hipError_t launch_pack_idx(const float* src, int64_t n, uint8_t* codes,
                           uint8_t* scales, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_idx_kernel, dim3(grid_for(n * 4, 256)), dim3(256), 0,
                     s, src, n, codes, scales);
  return hipGetLastError();
}

hipError_t launch_pack_swa(const float* src, int64_t n, uint8_t* codes,
                           hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t n4 = n * 128;
  hipLaunchKernelGGL(pack_swa_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, s,
                     src, n4, reinterpret_cast<uint32_t*>(codes));
  return hipGetLastError();
}

hipError_t launch_unpack(int fmt, const uint8_t* codes, const uint8_t* scales,
                         int64_t n, float* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int bpr = fmt == 0 ? 256 : (fmt == 1 ? 64 : 512);
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(n * bpr, 256)), dim3(256), 0,
                     s, fmt, codes, scales, n, dst);
  return hipGetLastError();
}

hipError_t launch_block_keys(const uint8_t* codes, const uint8_t* scales,
                             int64_t n_cap, const int32_t* n_entries, int B,
                             int block, uint16_t* keys, hipStream_t s) {
  const int64_t nb = (n_cap + block - 1) / block;
  const int64_t total = (int64_t)B * nb * 128;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(block_keys_kernel, dim3(grid_for(total, 256)), dim3(256),
                     0, s, codes, scales, n_cap, n_entries, nb, block, keys,
                     total);
  return hipGetLastError();
}

hipError_t launch_nblocks(const int32_t* n_entries, int B, int block,
                          int32_t* nblk, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(nblocks_kernel, dim3((unsigned)((B + 255) / 256)),
                     dim3(256), 0, s, n_entries, B, block, nblk);
  return hipGetLastError();
}

}  // namespace csa2
