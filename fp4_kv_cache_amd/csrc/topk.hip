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
// Tile pruning.  Rows are cut into 32-element tiles and each tile's largest
// score is known (the indexer writes it; tilemax_kernel computes it for a
// plain score array).  Let M be the k-th largest tile maximum: k different
// tiles each hold an element >= M, so the k-th largest score is >= M, and
// every top-k element lies in a tile whose maximum is >= M.  One 512-thread
// workgroup per row therefore (1) finds M by selecting the top-k tile
// maxima, (2) lists, in order, every tile whose maximum is >= M (about k
// tiles), and (3) selects the top-k among those tiles' scores only.  Rows
// short enough for one pass skip the pruning.  Each selection streams its
// input through block_select in passes of 16,384 register-held keys, keeping
// the running winners (in id order) in LDS.
#include <math.h>

#include "common.h"
#include "internal.h"
#include "select.h"

namespace csa2 {
namespace {

constexpr int kNT = 512;                    // threads per row
constexpr int kPer = 32;                    // keys per thread
constexpr int kCap = kNT * kPer;            // 16384 keys per pass
constexpr int kNB = 2048;
constexpr int kTileList = 4096;             // candidate tiles held in LDS
static_assert(kNB >= 2048, "winners (k <= 2048) are staged in the histogram");

struct RowSmem {
  uint32_t key[kCap];
  int32_t id[kCap];
  int32_t tiles[kTileList];
  SelSmem<kNT, kNB> sel;
};

// Top-k of the `count` (key, id) pairs held in sm.key/sm.id (ids in
// order): the winners are compacted, still in id order, to the front.
// Returns their number.  PER keys per thread; count <= kNT * PER.
template <int PER>
__device__ __forceinline__ int select_dense(RowSmem& sm, int count, int k) {
  const int tid = threadIdx.x;
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int pos = tid * PER + j;
    key[j] = pos < count ? sm.key[pos] : 0u;
  }
  const SelResult r = block_select<kNT, PER, kNB>(key, k, sm.sel);
  int tot;
  int p = sel_excl_scan<kNT, kNB>(__popc(r.mask), tot, sm.sel);
  // In-order compaction of the winners (at most k <= kNB): keys come from
  // registers; ids are staged through the histogram buffer (free after the
  // selection) so no thread overwrites an id another has yet to read.
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (r.mask & (1u << j)) {
      sm.sel.hist[p] = sm.id[tid * PER + j];
      sm.key[p] = key[j];
      ++p;
    }
  __syncthreads();
  for (int q = tid; q < tot; q += kNT) sm.id[q] = sm.sel.hist[q];
  __syncthreads();
  return tot;
}

__device__ __forceinline__ int select_any(RowSmem& sm, int count, int k) {
  if (count <= kNT * 2) return select_dense<2>(sm, count, k);
  if (count <= kNT * 8) return select_dense<8>(sm, count, k);
  return select_dense<kPer>(sm, count, k);
}

// Streaming top-k into LDS: feeds src.load(i, value, id) for i < n (ids ascending
// in i) through passes of up to kCap keys; afterwards key/id[0..count) hold
// the winners in id order.
template <typename Src>
__device__ __forceinline__ int stream_select(RowSmem& sm, int64_t n, int k,
                                             Src src) {
  const int tid = threadIdx.x;
  int count = 0;
  int64_t pos = 0;
  bool first = true;
  while (first || pos < n) {
    first = false;
    // Fill the free slots after the current winners: loads of a half pass
    // are all issued before their stores.
    const int64_t room = kCap - count;
    const int fill = (int)(n - pos < room ? n - pos : room);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      constexpr int kH = kCap / kNT / 2;
      float fv[kH];
      int32_t fi[kH];
#pragma unroll
      for (int j = 0; j < kH; ++j) {
        // Unconditional raw loads from a clamped index (n >= 1 whenever
        // fill > 0); keys are formed only after every load is issued.
        const int s = (h * kH + j) * kNT + tid;
        int64_t i = pos + (s - count);
        i = i < 0 ? 0 : (i >= n ? (n > 0 ? n - 1 : 0) : i);
        src.load(i, fv[j], fi[j]);
      }
#pragma unroll
      for (int j = 0; j < kH; ++j) {
        const int s = (h * kH + j) * kNT + tid;
        if (s >= count && s < count + fill) {
          sm.key[s] = fi[j] >= 0 ? score_key(fv[j]) : 0u;
          sm.id[s] = fi[j];
        }
      }
    }
    pos += fill;
    __syncthreads();
    count = select_any(sm, count + fill, k);
  }
  return count;
}

// Element sources for stream_select (ids ascending in i): load(i, v, id)
// reads the raw value and id of element i (always a valid index).
template <bool HAS_IDS>
struct ScoreSrc {                 // a score row; ids = positions or ids[]
  const float* row;
  const int32_t* idrow;
  __device__ __forceinline__ void load(int64_t i, float& v, int32_t& id) const {
    v = row[i];
    id = HAS_IDS ? idrow[i] : (int32_t)i;
  }
};
struct TileSrc {                  // tile maxima; ids = tile numbers
  const float* trow;
  __device__ __forceinline__ void load(int64_t t, float& v, int32_t& id) const {
    v = trow[t];
    id = (int32_t)t;
  }
};

struct RowArgs {
  const float* scores;      // row stride ld
  const float* tmax;        // nullable; row stride ceil(ld / 32)
  int64_t ld;
  const int32_t* n_valid;   // nullable
  const int32_t* ids;       // nullable
  int k;
  int block;
  const int32_t* limit;     // nullable
  int32_t* out;             // [B][k * block]
};

template <bool HAS_IDS>
__global__ __launch_bounds__(kNT) void row_select_kernel(RowArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  RowSmem& sm = *reinterpret_cast<RowSmem*>(smem_raw);
  const int b = blockIdx.x, tid = threadIdx.x;
  int64_t len = a.ld;
  if (a.n_valid) {
    const int64_t nv = a.n_valid[b];
    len = nv < len ? (nv > 0 ? nv : 0) : len;
  }
  const ScoreSrc<HAS_IDS> from_scores{
      a.scores + (int64_t)b * a.ld, HAS_IDS ? a.ids + (int64_t)b * a.ld : nullptr};
  const int64_t n_t = (len + 31) >> 5;
  int count = 0;
  bool pruned = a.tmax != nullptr && n_t > a.k;
  if (pruned) {
    const float* trow = a.tmax + (int64_t)b * ((a.ld + 31) >> 5);
    // (1) M = the k-th largest tile maximum.
    const int ct = stream_select(sm, n_t, a.k, TileSrc{trow});
    uint32_t mk = 0xFFFFFFFFu, dummy = 0u;
    for (int p = tid; p < ct; p += kNT) mk = min(mk, sm.key[p]);
    sel_minmax<kNT, kNB>(mk, dummy, sm.sel);
    // (2) every tile whose maximum is >= M, in order (each thread scans a
    // run of kPer tiles).
    int n_list = 0;
    for (int64_t t0 = 0; t0 < n_t; t0 += kCap) {
      const int64_t tb = t0 + (int64_t)tid * kPer;
      uint32_t fl = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (tb + j < n_t && score_key(trow[tb + j]) >= mk) fl |= 1u << j;
      int tot;
      int p = sel_excl_scan<kNT, kNB>(__popc(fl), tot, sm.sel);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (fl & (1u << j)) {
          if (n_list + p < kTileList) sm.tiles[n_list + p] = (int32_t)(tb + j);
          ++p;
        }
      n_list += tot;
    }
    __syncthreads();
    // (3) the elements >= M of the listed tiles, densely, in id order.
    if (n_list <= kTileList) {
      int n_c = 0;
      for (int l0 = 0; l0 < n_list; l0 += kNT) {
        const int l = l0 + tid;
        const bool have = l < n_list;
        const int64_t base = (int64_t)(have ? sm.tiles[l] : 0) * 32;
        float vv[32];
        int32_t ii[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int64_t pos = base + j < len ? base + j : len - 1;   // len >= 1
          from_scores.load(pos, vv[j], ii[j]);
        }
        uint32_t kk[32];
        uint32_t fl = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          kk[j] = ii[j] >= 0 ? score_key(vv[j]) : 0u;
          if (have && base + j < len && kk[j] >= mk) fl |= 1u << j;
        }
        int tot;
        int p = sel_excl_scan<kNT, kNB>(__popc(fl), tot, sm.sel);
        if (n_c + tot <= kCap) {
#pragma unroll
          for (int j = 0; j < 32; ++j)
            if (fl & (1u << j)) {
              sm.key[n_c + p] = kk[j];
              sm.id[n_c + p] = ii[j];
              ++p;
            }
        }
        n_c += tot;
      }
      __syncthreads();
      if (n_c <= kCap) count = select_any(sm, n_c, a.k);
      else pruned = false;     // (massive ties) fall back to a full pass
    } else {
      pruned = false;
    }
  }
  if (!pruned) count = stream_select(sm, len, a.k, from_scores);
  // Winners in id order -> out[b], expanded by `block` and clipped.
  const int64_t ob = (int64_t)b * a.k * a.block;
  const int64_t lim = a.limit ? (int64_t)a.limit[b] : INT64_MAX;
  for (int p = tid; p < count; p += kNT) {
    const int64_t id = sm.id[p];
    for (int t = 0; t < a.block; ++t) {
      const int64_t q = id * a.block + t;
      a.out[ob + (int64_t)p * a.block + t] = q < lim ? (int32_t)q : -1;
    }
  }
  for (int64_t p = (int64_t)count * a.block + tid; p < (int64_t)a.k * a.block;
       p += kNT)
    a.out[ob + p] = -1;
}

// Tile maxima of a plain score array (entries with a negative id count as
// -inf).  One thread per tile.
__global__ void tilemax_kernel(const float* __restrict__ scores, int64_t ld,
                               const int32_t* __restrict__ ids, int B,
                               float* __restrict__ tmax) {
  const int64_t nt = (ld + 31) >> 5;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nt * B) return;
  const int64_t b = t / nt, tt = t % nt;
  float mx = -__builtin_inff();
  for (int j = 0; j < 32; ++j) {
    const int64_t i = tt * 32 + j;
    if (i >= ld) break;
    const float v = scores[b * ld + i];
    if ((!ids || ids[b * ld + i] >= 0) && v > mx) mx = v;
  }
  tmax[t] = mx;
}

}  // namespace

size_t topk_workspace(int B, int64_t ld) {
  if (ld <= kCap) return 0;
  return (((size_t)B * ((ld + 31) >> 5) * 4) + 255) & ~size_t(255);
}

hipError_t launch_row_select(const float* scores, const float* tmax,
                             int64_t ld, const int32_t* n_valid,
                             const int32_t* ids, int B, int k, int block,
                             const int32_t* limit, int32_t* out,
                             hipStream_t s) {
  if (B == 0) return hipSuccess;
  static std::atomic<uint64_t> lds_set0{0}, lds_set1{0};
  hipError_t e = ensure_lds_limit(
      reinterpret_cast<const void*>(row_select_kernel<false>),
      (int)sizeof(RowSmem), lds_set0);
  if (e != hipSuccess) return e;
  e = ensure_lds_limit(reinterpret_cast<const void*>(row_select_kernel<true>),
                       (int)sizeof(RowSmem), lds_set1);
  if (e != hipSuccess) return e;
  RowArgs a{};
  a.scores = scores;
  a.tmax = tmax;
  a.ld = ld;
  a.n_valid = n_valid;
  a.ids = ids;
  a.k = k;
  a.block = block;
  a.limit = limit;
  a.out = out;
  if (ids)
    hipLaunchKernelGGL(row_select_kernel<true>, dim3((unsigned)B), dim3(kNT),
                       sizeof(RowSmem), s, a);
  else
    hipLaunchKernelGGL(row_select_kernel<false>, dim3((unsigned)B), dim3(kNT),
                       sizeof(RowSmem), s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid,
                       const int32_t* ids, int B, int k, int block,
                       const int32_t* limit, int32_t* out, void* ws,
                       hipStream_t s) {
  if (B == 0) return hipSuccess;
  float* tmax = nullptr;
  if (ld > kCap) {
    tmax = static_cast<float*>(ws);
    const int64_t n = (int64_t)B * ((ld + 31) >> 5);
    hipLaunchKernelGGL(tilemax_kernel, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, scores, ld, ids, B, tmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_row_select(scores, tmax, ld, n_valid, ids, B, k, block, limit,
                           out, s);
}

}  // namespace csa2
