// Device-side types and helpers shared by the libcsa2 kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMainDim = 512;     // main latent width
constexpr int kMainCodeBytes = 256;
constexpr int kMainScaleBytes = 32;
constexpr int kIdxDim = 128;      // indexer head width
constexpr int kIdxCodeBytes = 64;
constexpr int kIdxScaleBytes = 4;
constexpr int kIdxHeads = 32;
constexpr int kHeads = 64;        // attention query heads
constexpr int kWindow = 128;      // sliding-window rows per sequence

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// E8M0 code -> float32 2^(c-127) (code 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  return c == 0 ? u2f(0x00400000u) : u2f(c << 23);
}

// Bit-reinterpret helpers between packed bf16 pairs and uint32.
__device__ __forceinline__ uint32_t bf2_bits(bf16x2 v) {
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16x8 bits_to_bf8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Selection key of a score: an order-preserving map float32 -> uint32
// (larger score -> larger key) with NaN and -inf -> 0 (never chosen) and
// -0 -> key(+0), so equal scores have equal keys.  Selects only, no
// branches.
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t u = f2u(v);
  u = (u << 1) ? u : 0u;                                   // -0 -> +0
  const uint32_t key = (int32_t)u < 0 ? ~u : (u | 0x80000000u);
  return v > -__builtin_inff() ? key : 0u;
}

// Raise a kernel's dynamic-LDS limit once per device (host side).
inline hipError_t ensure_lds_limit(const void* func, int bytes,
                                   std::atomic<uint64_t>& done_mask) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done_mask.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done_mask.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace csa2
