// Cache write path: FP4 main-KV, MXFP4 indexer-key and E4M3 window packing,
// exact dequantisation, and pooled bf16 block keys.
//
// Sources: "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
// (mer.run) section 5, quantiser equation s_g = E4M3(max|x|/6),
// x_i -> E2M1(x_i/s_g), and section 2 (288 B / 68 B entries);
// "DeepSeek-V4.1-Flash, 2. Architecture" section 2.4.4 (E2M1 + one E4M3
// scale per 16 channels, no global scale; MXFP4 indexer keys; FP8 window).
// The exact quantisers themselves are in quant.h.
#include "common.h"
#include "internal.h"
#include "quant.h"

namespace csa2 {
namespace {

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
  uint32_t w[2], sc;
  quant_main_group(x, w, sc);
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
  uint32_t w[4], sb;
  quant_idx_block(x, w, sb);
  *reinterpret_cast<uint4*>(codes + row * 64 + blk * 16) =
      make_uint4(w[0], w[1], w[2], w[3]);
  scales[row * 4 + blk] = (uint8_t)sb;
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

}  // namespace csa2
