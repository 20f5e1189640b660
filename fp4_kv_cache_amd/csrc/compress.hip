// CSA2 write path at decode time: main-KV projection, sequence compression,
// indexer-key projection, and the append into the FP4 / MXFP4 / E4M3 caches.
//
// Sources: "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
// (mer.run) section 4.1 equations: C = H W^KV, Z = H W^Z (both 512 wide);
// C_bar_j = sum over the block B_j of softmax(Z_i) (.) C_i, blocks of m
// tokens without overlap; K^I_j = C_bar_j W^IK; section 5 and "DeepSeek-V4.1-
// Flash, 2. Architecture" 2.3 / 2.4.4 for the cache formats (the window keeps
// the uncompressed rows C_i in E4M3).
//
// gfx950 mapping.  The two projections are one skinny GEMM: M = B*m hidden
// rows, K = d, N = 1024 (the W^KV columns, then the W^Z columns).  At
// decode M is small and the GEMM is bound by streaming the bf16 weights
// (14.7 MB at d = 7168), so a workgroup owns 32 output columns and one
// slice of 1,024 reduction values, its 8 wavefronts split the slice, and
// their v_mfma_f32_32x32x16_bf16 accumulators (A = 32 hidden rows, B = 32
// weight rows: the weights are [out][in], so every lane's 8 k-values are one
// 16-byte load) are summed through LDS.  The slice partials are summed in a
// fixed order by the epilogue, so results are bitwise deterministic.  The
// epilogue (one workgroup per sequence) forms C and Z, the per-channel
// softmax pooling over the m tokens, K^I, and writes the new entry with the
// exact quantisers of quant.h.
#include "common.h"
#include "internal.h"
#include "quant.h"

namespace csa2 {
namespace {

constexpr int kN = 1024;            // C columns, then Z columns
constexpr int kCols = 32;           // output columns per workgroup
constexpr int kWaves = 8;           // wavefronts per workgroup
constexpr int kSteps = 8;           // 16-wide k-steps per wavefront
constexpr int kSliceSteps = kWaves * kSteps;   // k-steps per slice
constexpr int kMChunk = 64;         // hidden rows per pass (two 32-row tiles)
constexpr int kMaxM = 16;           // tokens per block
constexpr int kMaxS = 16;           // slices at d = 16384

__host__ __device__ constexpr int n_slices(int d) {
  return (d / 16 + kSliceSteps - 1) / kSliceSteps;
}

// Workgroup (column tile, slice): 32 output columns over the slice's 64
// k-steps; wavefront w takes k-steps 8w .. 8w+7 of the slice.  All of a
// wavefront's loads are issued before its matrix ops (one memory latency
// per pass, not one per k-step): a scheduling barrier keeps the compiler
// from interleaving them with the matrix ops, which left about one load in
// flight per wavefront.  Its weight operands stay in registers across the
// 64-row passes over the hidden rows.  k-steps past the end (only in the
// last slice) read a clamped step and enter as zero operands, set after the
// pass's loads are issued, since the test waits for the weights.
__global__ __launch_bounds__(kWaves * 64) void compress_gemm_kernel(
    const uint16_t* __restrict__ h, int M, int d,
    const uint16_t* __restrict__ w_kv, const uint16_t* __restrict__ w_z,
    float* __restrict__ part) {
  __shared__ float red[kWaves][kMChunk][kCols + 1];
  const int col0 = blockIdx.x * kCols;
  const int slice = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, kg = lane >> 5;
  const uint16_t* W = col0 < 512 ? w_kv + (int64_t)col0 * d
                                 : w_z + (int64_t)(col0 - 512) * d;
  const int nks = d / 16;
  const int ks0 = slice * kSliceSteps + wave * kSteps;
  int kofs[kSteps];
  bool kin[kSteps];
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    const int ks = ks0 + j;
    kin[j] = ks < nks;
    kofs[j] = 16 * (kin[j] ? ks : nks - 1) + 8 * kg;
  }
  const uint16_t* wrow = W + (int64_t)r * d;
  bf16x8 bw[kSteps];
#pragma unroll
  for (int j = 0; j < kSteps; ++j)
    bw[j] = *reinterpret_cast<const bf16x8*>(wrow + kofs[j]);
  const bool ragged = ks0 + kSteps > nks;     // wavefront-uniform
  for (int m0 = 0; m0 < M; m0 += kMChunk) {
    // Rows past M read a clamped row; their results are never stored.
    const int ra = m0 + r < M ? m0 + r : M - 1;
    const int rb = m0 + 32 + r < M ? m0 + 32 + r : M - 1;
    const uint16_t* ha = h + (int64_t)ra * d;
    const uint16_t* hb = h + (int64_t)rb * d;
    bf16x8 a0[kSteps], a1[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      a0[j] = *reinterpret_cast<const bf16x8*>(ha + kofs[j]);
      a1[j] = *reinterpret_cast<const bf16x8*>(hb + kofs[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ragged) {
#pragma unroll
      for (int j = 0; j < kSteps; ++j)
        if (!kin[j]) bw[j] = bf16x8{};
    }
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[j], bw[j], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[j], bw[j], acc1, 0, 0, 0);
    }
    // Lane l holds column r of rows 8a + 4kg + q (q < 4) of each tile.
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        red[wave][8 * a + 4 * kg + q][r] = acc0[4 * a + q];
        red[wave][32 + 8 * a + 4 * kg + q][r] = acc1[4 * a + q];
      }
    __syncthreads();
    for (int i = threadIdx.x; i < kMChunk * kCols; i += kWaves * 64) {
      const int row = i / kCols, c = i % kCols;
      if (m0 + row < M) {
        float v = red[0][row][c];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += red[w][row][c];
        __builtin_nontemporal_store(
            v, &part[((int64_t)slice * M + m0 + row) * kN + col0 + c]);
      }
    }
    // The next pass reuses `red` (no barrier after the last pass: one
    // behind global stores would hold every wavefront until they land).
    if (m0 + kMChunk < M) __syncthreads();
  }
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Four workgroups of 512 threads per sequence (blockIdx.y = j), thread c
// owning channel c: each forms the pooled row C_bar and computes MX block j
// of K^I (outputs 32j .. 32j+31); workgroup 0 also writes the main entry
// and the window rows.  Everything a workgroup reads -- the slice partials
// of its channels and its 32 rows of W^IK (thread c: 32 weights of output
// 32j + c/16) -- is requested at the start, so it waits for memory about
// once.  MT: a bound on m known at compile time (the tokens' loads
// unrolled), or 0 for a loop over tokens; SMAX: a bound on the slice count
// (8 up to d = 8192), so no more loads are issued than there are slices.
template <int MT, int SMAX>
__global__ __launch_bounds__(512) void compress_epilogue_kernel(
    const float* __restrict__ part, int M, int m, int S,
    const uint16_t* __restrict__ w_ik, const int32_t* __restrict__ rows,
    int64_t n_cap, uint8_t* __restrict__ main_codes,
    uint8_t* __restrict__ main_scales, uint8_t* __restrict__ idx_codes,
    uint8_t* __restrict__ idx_scales, uint8_t* __restrict__ swa,
    const int32_t* __restrict__ swa_slot, float* __restrict__ cbar_out,
    float* __restrict__ ki_out, float* __restrict__ c_out) {
  __shared__ __align__(16) float cbar[512];
  __shared__ float kpart[512];
  const int b = blockIdx.x, j = blockIdx.y, c = threadIdx.x;
  const bool lead = j == 0;                 // writes the main entry, window
  const int o = 32 * j + (c >> 4), sx = c & 15;   // output, its sixteenth
  const u32x4* wr =
      reinterpret_cast<const u32x4*>(w_ik + (int64_t)o * 512 + 32 * sx);
  u32x4 wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = wr[i];
  const int slot = swa != nullptr ? swa_slot[b] : 0;

  // C and Z of this channel for each token: the slices summed in order.
  // Every slice's load is issued unconditionally (slices past S read slice
  // S-1 and are not summed), so they are all in flight at once.
  float cv[kMaxM], zv[kMaxM];
  auto token = [&](int i) {
    const int64_t row = (int64_t)b * m + i;
    float pc[SMAX], pz[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int sl = s < S ? s : S - 1;
      const int64_t at = ((int64_t)sl * M + row) * kN + c;
      pc[s] = part[at];
      pz[s] = part[at + 512];
    }
    float cs = 0.0f, zs = 0.0f;
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (s < S) { cs += pc[s]; zs += pz[s]; }
    cv[i] = cs;
    zv[i] = zs;
  };
  if constexpr (MT > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (i < m) token(i);
  } else {
    for (int i = 0; i < m; ++i) token(i);
  }
  // softmax over the block's m tokens
  float zmax = -__builtin_inff();
  for (int i = 0; i < m; ++i) zmax = fmaxf(zmax, zv[i]);
  float num = 0.0f, den = 0.0f;
  for (int i = 0; i < m; ++i) {
    const float e = expf(zv[i] - zmax);
    num += e * cv[i];
    den += e;
  }
  const float v = num / den;
  cbar[c] = v;
  if (lead) {
    if (cbar_out) cbar_out[(int64_t)b * 512 + c] = v;
    for (int i = 0; i < m; ++i) {
      if (c_out) c_out[((int64_t)b * m + i) * 512 + c] = cv[i];
      if (swa) {
        const int w = ((slot + i) % kWindow + kWindow) % kWindow;
        swa[((int64_t)b * kWindow + w) * 512 + c] =
            (uint8_t)e4m3_from_f64((double)cv[i]);
      }
    }
  }
  __syncthreads();
  // K^I = C_bar W^IK: a sixteenth of output o's dot per thread (channels
  // 32sx .. 32sx+31, as four chains of eight summed in a fixed order), then
  // the sixteen in order.
  float ac[4];
  const float4* cb4 = reinterpret_cast<const float4*>(cbar + 32 * sx);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 x0 = cb4[2 * i], x1 = cb4[2 * i + 1];
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a += bf16_bits_to_f32(wv[i][e] & 0xFFFFu) * xs[2 * e];
      a += bf16_bits_to_f32(wv[i][e] >> 16) * xs[2 * e + 1];
    }
    ac[i] = a;
  }
  kpart[c] = (ac[0] + ac[1]) + (ac[2] + ac[3]);
  __syncthreads();
  const int64_t row = rows[b];
  const bool ok = row >= 0 && row < n_cap;   // other rows are not written
  const int64_t er = (int64_t)b * n_cap + row;
  // The append, one value per thread (the same arithmetic as
  // quant_main_group / quant_idx_block, spread over lanes): a group's
  // amax over its lanes, each lane's code, and 8 codes OR-ed into a word.
  auto or8 = [](uint32_t x) {
    x |= __shfl_xor(x, 1);
    x |= __shfl_xor(x, 2);
    return x | __shfl_xor(x, 4);
  };
  if (lead) {
    // Main row: channel c in group c / 16 (16 lanes of one wavefront).
    const float x = cbar[c];
    float amax = fabsf(x);
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
    const uint32_t sc = e4m3_from_f64((double)amax / 6.0);
    const float sg = e4m3_to_f32(sc);
    const uint32_t code = sg > 0.0f ? e2m1_code_scaled(x, sg)
                                    : (signbit(x) ? 8u : 0u);
    const uint32_t word = or8(code << (4 * (c & 7)));
    if (ok && (c & 7) == 0)
      *reinterpret_cast<uint32_t*>(main_codes + er * 256 + 4 * (c >> 3)) = word;
    if (ok && (c & 15) == 0) main_scales[er * 32 + (c >> 4)] = (uint8_t)sc;
  }
  if (c < 32) {                           // lanes of wavefront 0
    // Indexer key: output 32j + c of MX block j.
    float x = kpart[16 * c];
#pragma unroll
    for (int i = 1; i < 16; ++i) x += kpart[16 * c + i];
    float amax = fabsf(x);
#pragma unroll
    for (int sh = 1; sh < 32; sh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
    int e = -127;
    if (amax > 0.0f) {
      e = ilogb((double)amax) - 2;          // largest E2M1 exponent is 2
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    const uint32_t code = e2m1_code_f64((double)x * ldexp(1.0, -e));
    const uint32_t word = or8(code << (4 * (c & 7)));
    if (ok && (c & 7) == 0)
      *reinterpret_cast<uint32_t*>(idx_codes + er * 64 + 16 * j + 4 * (c >> 3)) = word;
    if (ok && c == 0) idx_scales[er * 4 + j] = (uint8_t)(e + 127);
    if (ki_out) ki_out[(int64_t)b * 128 + 32 * j + c] = x;
  }
}

}  // namespace

size_t compress_workspace(int B, int m, int d) {
  return (((size_t)n_slices(d) * B * m * kN * 4) + 255) & ~size_t(255);
}

hipError_t launch_compress(const uint16_t* h, int B, int m, int d,
                           const uint16_t* w_kv, const uint16_t* w_z,
                           const uint16_t* w_ik, const int32_t* rows,
                           int64_t n_cap, uint8_t* main_codes,
                           uint8_t* main_scales, uint8_t* idx_codes,
                           uint8_t* idx_scales, uint8_t* swa,
                           const int32_t* swa_slot, float* cbar_out,
                           float* ki_out, float* c_out, void* ws,
                           hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (m < 1 || m > kMaxM || d < 16 || d % 16) return hipErrorInvalidValue;
  const int M = B * m;
  const int S = n_slices(d);
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(compress_gemm_kernel, dim3(kN / kCols, S),
                     dim3(kWaves * 64), 0, s, h, M, d, w_kv, w_z, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto epi = S <= 8 ? (m <= 2   ? compress_epilogue_kernel<2, 8>
                       : m <= 4 ? compress_epilogue_kernel<4, 8>
                                : compress_epilogue_kernel<0, 8>)
                    : (m <= 2   ? compress_epilogue_kernel<2, kMaxS>
                       : m <= 4 ? compress_epilogue_kernel<4, kMaxS>
                                : compress_epilogue_kernel<0, kMaxS>);
  hipLaunchKernelGGL(epi, dim3((unsigned)B, 4), dim3(512), 0, s, part, M, m, S,
                     w_ik, rows, n_cap, main_codes, main_scales, idx_codes,
                     idx_scales, swa, swa_slot, cbar_out, ki_out, c_out);
  return hipGetLastError();
}

}  // namespace csa2
