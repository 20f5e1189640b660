// Exact top-k selection per row, with the pool expansion of the
// hierarchical indexer.
//
// Sources: "DeepSeek-V4: Towards Highly Efficient Million-Token Context
// Intelligence" (baisen.site), CSA step 2 top-k equation; "DeepSeek-V4.1-Flash:
// Pushing the Limits of KV Cache Compression" (mer.run) section 4.1
// (S_t = Top512) and section 4.3 (top-2048 blocks, union of their 8
// positions).  The pages give no tie rule; here a higher score wins and
// equal scores go to the lower id.
//
// Design.  A row is cut into segments of at most kChunk elements; one
// 1024-thread workgroup selects the exact top-k of a segment entirely in
// LDS, and the survivors of all segments (still in id order) are selected
// again until one segment remains.  The union of per-segment top-k sets
// contains the row's top-k, so the result is exact.
//
// Inside a segment the k-th value is found by narrowing a value interval
// [lo, hi] that holds it: the candidates in the interval are binned by a
// linear, monotone map of their value into 2048 bins (LDS atomics; a linear
// map spreads the data, so few lanes collide on a bin), a block scan finds
// the bin where the running count from the top reaches the number still
// needed, and the interval shrinks to that bin's actual minimum and maximum.
// Each pass shrinks the interval at least 2048-fold, so it ends after a few
// passes either with the bin holding exactly the number needed or with all
// candidates equal (then the lowest ids win).  The chosen elements are then
// written in id order with a block-wide prefix sum.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kChunk = 16384;               // max elements per segment
constexpr int kPer = kChunk / kThreads;     // elements per thread
constexpr int kBins = 2048;
constexpr int kWavesTk = kThreads / 64;

struct TkSmem {
  float v[kChunk];
  int32_t id[kChunk];
  int32_t hist[kBins];
  int32_t red[kWavesTk];
  float fred[2][kWavesTk];
  int32_t bstar, cum_before;
};

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Block-wide exclusive prefix sum; also returns the block total.
__device__ __forceinline__ int block_excl_scan(int x, int& total, TkSmem& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) sm.red[wv] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWavesTk; ++i) {
    const int t = sm.red[i];
    before += i < wv ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

__device__ __forceinline__ void block_minmax(float& mn, float& mx, TkSmem& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) { sm.fred[0][wv] = mn; sm.fred[1][wv] = mx; }
  __syncthreads();
  mn = sm.fred[0][0];
  mx = sm.fred[1][0];
#pragma unroll
  for (int i = 1; i < kWavesTk; ++i) {
    mn = fminf(mn, sm.fred[0][i]);
    mx = fmaxf(mx, sm.fred[1][i]);
  }
  __syncthreads();
}

__device__ __forceinline__ int bin_of(float v, float hi, double inv) {
  const double x = ((double)hi - (double)v) * inv;
  return x >= (double)(kBins - 1) ? kBins - 1 : (int)x;
}

struct TkArgs {
  const float* vals;        // input values, row stride ld
  const int32_t* ids;       // nullable: ids = positions
  int64_t ld;
  const int32_t* n_valid;   // nullable (rows then have length `len`)
  int64_t len;              // row length at this stage
  int seg_len;
  int segs;                 // segments per row at this stage
  int k;
  // intermediate output: [B][segs][k]
  float* out_vals;
  int32_t* out_ids;
  // final output (when segs == 1): [B][k * block]
  int32_t* out;
  int block;
  const int32_t* limit;
};

__global__ __launch_bounds__(kThreads) void topk_kernel(TkArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TkSmem& sm = *reinterpret_cast<TkSmem*>(smem_raw);
  const int seg = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int64_t row_len = a.len;
  if (a.n_valid) {
    const int64_t nv = a.n_valid[b];
    row_len = nv < row_len ? (nv > 0 ? nv : 0) : row_len;
  }
  const int64_t s0 = (int64_t)seg * a.seg_len;
  int64_t s1 = s0 + a.seg_len;
  if (s1 > row_len) s1 = row_len;
  const float NEG = -__builtin_inff();

  // 1. Coalesced load into LDS; invalid elements become -inf.
  for (int j = 0; j < kPer; ++j) {
    const int li = j * kThreads + tid;
    const int64_t gi = s0 + li;
    float v = NEG;
    int32_t id = -1;
    if (gi < s1) {
      v = a.vals[(int64_t)b * a.ld + gi];
      id = a.ids ? a.ids[(int64_t)b * a.ld + gi] : (int32_t)gi;
      if (!(v > NEG) || id < 0) v = NEG;     // NaN, -inf, bad id
    }
    sm.v[li] = v;
    sm.id[li] = id;
  }
  __syncthreads();

  // 2. Each thread owns a contiguous run of kPer elements.
  float vr[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) vr[j] = sm.v[tid * kPer + j];
  int nval = 0;
  float mn = __builtin_inff(), mx = NEG;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (vr[j] > NEG) { ++nval; mn = fminf(mn, vr[j]); mx = fmaxf(mx, vr[j]); }
  int total_valid;
  block_excl_scan(nval, total_valid, sm);
  block_minmax(mn, mx, sm);

  // 3. Narrow [lo, hi] until the selection is decided.
  // Selected: v > hi, plus -- if take_all -- every v in [lo, hi], else (all
  // candidates equal) the first `need` of them in id order.
  float lo = mn, hi = mx;
  int need = a.k;
  bool take_all = true;
  if (total_valid > a.k) {
    take_all = false;
    for (int it = 0; it < 64; ++it) {
      if (!(lo < hi)) break;                   // all candidates tie
      for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0;
      __syncthreads();
      const double inv = (double)kBins / ((double)hi - (double)lo);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (vr[j] >= lo && vr[j] <= hi) atomicAdd(&sm.hist[bin_of(vr[j], hi, inv)], 1);
      __syncthreads();
      const int h0 = sm.hist[2 * tid], h1 = sm.hist[2 * tid + 1];
      int tot;
      const int ex = block_excl_scan(h0 + h1, tot, sm);
      if (ex < need && ex + h0 + h1 >= need) {
        if (ex + h0 >= need) { sm.bstar = 2 * tid; sm.cum_before = ex; }
        else { sm.bstar = 2 * tid + 1; sm.cum_before = ex + h0; }
      }
      __syncthreads();
      const int bs = sm.bstar;
      const int cnt = sm.hist[bs];
      need -= sm.cum_before;
      float bmn = __builtin_inff(), bmx = NEG;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (vr[j] >= lo && vr[j] <= hi && bin_of(vr[j], hi, inv) == bs) {
          bmn = fminf(bmn, vr[j]);
          bmx = fmaxf(bmx, vr[j]);
        }
      block_minmax(bmn, bmx, sm);
      lo = bmn;
      hi = bmx;
      if (cnt == need) { take_all = true; break; }
    }
  }

  // 4. Flags, ranks among ties, and the in-order compaction.
  int ntie = 0;
  if (!take_all) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) ntie += (vr[j] == lo) ? 1 : 0;
  }
  int tie_total;
  int tie_rank = block_excl_scan(ntie, tie_total, sm);
  uint32_t selmask = 0;
  int nsel = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    bool s;
    if (!(vr[j] > NEG)) s = false;
    else if (take_all) s = vr[j] >= lo;
    else if (vr[j] > hi) s = true;
    else if (vr[j] == lo) { s = tie_rank < need; ++tie_rank; }
    else s = false;
    if (s) { selmask |= 1u << j; ++nsel; }
  }
  int nsel_total;
  int pos = block_excl_scan(nsel, nsel_total, sm);

  const bool final_stage = a.segs == 1;
  if (!final_stage) {
    const int64_t ob = ((int64_t)b * a.segs + seg) * a.k;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (selmask & (1u << j)) {
        a.out_vals[ob + pos] = vr[j];
        a.out_ids[ob + pos] = sm.id[tid * kPer + j];
        ++pos;
      }
    for (int p = nsel_total + tid; p < a.k; p += kThreads) {
      a.out_vals[ob + p] = NEG;
      a.out_ids[ob + p] = -1;
    }
    return;
  }
  const int64_t ob = (int64_t)b * a.k * a.block;
  const int64_t lim = a.limit ? (int64_t)a.limit[b] : INT64_MAX;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (selmask & (1u << j)) {
      const int64_t id = sm.id[tid * kPer + j];
      for (int t = 0; t < a.block; ++t) {
        const int64_t p = id * a.block + t;
        a.out[ob + (int64_t)pos * a.block + t] = p < lim ? (int32_t)p : -1;
      }
      ++pos;
    }
  for (int64_t p = (int64_t)nsel_total * a.block + tid; p < (int64_t)a.k * a.block;
       p += kThreads)
    a.out[ob + p] = -1;
}

}  // namespace

TopkPlan topk_plan(int64_t ld, int k) {
  TopkPlan p{};
  p.ld = ld;
  p.k = k;
  p.chunk = kChunk;
  int64_t len = ld;
  int st = 0;
  for (;;) {
    const int64_t segs = (len + kChunk - 1) / kChunk;
    p.len[st] = len;
    p.segs[st] = (int)(segs > 0 ? segs : 1);
    ++st;
    if (segs <= 1 || st >= 8) break;
    len = segs * (int64_t)k;
  }
  p.n_stages = st;
  return p;
}

size_t topk_workspace(int B, const TopkPlan& p) {
  size_t mx = 0;
  for (int s = 0; s + 1 < p.n_stages; ++s) {
    const size_t e = (size_t)B * p.segs[s] * p.k;
    if (e > mx) mx = e;
  }
  // two ping-pong buffers of (value, id) pairs, 256-byte aligned
  const size_t one = ((mx * 8) + 255) & ~size_t(255);
  return 2 * one;
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid,
                       const int32_t* ids, int B, int k, int block,
                       const int32_t* limit, int32_t* out, void* ws,
                       const TopkPlan& p, hipStream_t s) {
  if (B == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(topk_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(TkSmem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  size_t mx = 0;
  for (int st = 0; st + 1 < p.n_stages; ++st) {
    const size_t e = (size_t)B * p.segs[st] * p.k;
    if (e > mx) mx = e;
  }
  const size_t one = ((mx * 8) + 255) & ~size_t(255);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const float* in_vals = scores;
  const int32_t* in_ids = ids;
  int64_t in_ld = ld;
  for (int st = 0; st < p.n_stages; ++st) {
    TkArgs a{};
    a.vals = in_vals;
    a.ids = in_ids;
    a.ld = in_ld;
    a.n_valid = st == 0 ? n_valid : nullptr;
    a.len = p.len[st];
    a.seg_len = kChunk;
    a.segs = p.segs[st];
    a.k = k;
    uint8_t* buf = base + (st & 1) * one;
    a.out_vals = reinterpret_cast<float*>(buf);
    a.out_ids = reinterpret_cast<int32_t*>(buf + mx * 4);
    a.out = out;
    a.block = block;
    a.limit = limit;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.segs, (unsigned)B),
                       dim3(kThreads), sizeof(TkSmem), s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    in_vals = a.out_vals;
    in_ids = a.out_ids;
    in_ld = (int64_t)a.segs * k;
  }
  return hipSuccess;
}

}  // namespace csa2
