// Exact streaming top-k of one row inside one workgroup (device code), for
// any block size NT (a multiple of 256 threads).  Used by the row-select
// kernels and, as the exact fallback of the fused selection, by the
// attention kernel.
//
// Order as in select.h: a larger key first, equal keys by lower id.  The
// shared-memory type `Smem` has members key[NT * 16], id[NT * 16] and
// sel (SelSmem<NT, 256>); the winners so far stay at the front of key/id in
// id order while the rest of the row streams through in passes.
#pragma once
#include "common.h"
#include "select.h"

namespace csa2 {

constexpr int kStreamPer = 16;            // keys per thread in one pass

// Top-k of the `count` (key, id) pairs held in sm.key/sm.id (ids in
// order): the winners are compacted, still in id order, to the front.
// Returns their number.  PER keys per thread; count <= NT * PER.
template <int NT, int PER, typename Smem>
__device__ __forceinline__ int select_dense(Smem& sm, int count, int k) {
  static_assert(NT / 64 * 256 >= 2048, "staging room for 2048 winners");
  const int tid = threadIdx.x;
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {       // unconditional reads, then masks
    const int pos = tid * PER + j;
    const uint32_t kv = sm.key[pos];
    key[j] = pos < count ? kv : 0u;
  }
  const SelResult r = block_select<NT, PER, 256>(key, k, sm.sel);
  // In-order compaction of the winners (at most k <= 2048).  Every read of
  // sm.key finished inside the selection, so keys go straight to their
  // place; ids are staged through the (zero) histograms, which are cleared
  // again behind them.
  int32_t* stage = &sm.sel.hist[0][0];
  int32_t idv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) idv[j] = sm.id[tid * PER + j];
  int p = r.pos;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (r.mask & (1u << j)) {
      stage[p] = idv[j];
      sm.key[p] = key[j];
      ++p;
    }
  __syncthreads();
  for (int q = tid; q < r.total; q += NT) {
    sm.id[q] = stage[q];
    stage[q] = 0;
  }
  __syncthreads();
  return r.total;
}

template <int NT, typename Smem>
__device__ __forceinline__ int select_any(Smem& sm, int count, int k) {
  if (count <= NT * 2) return select_dense<NT, 2>(sm, count, k);
  if (count <= NT * 8) return select_dense<NT, 8>(sm, count, k);
  return select_dense<NT, kStreamPer>(sm, count, k);
}

// Streaming top-k into LDS: feeds src.load(i, value, id) for i < n (ids
// ascending in i) through passes of up to NT * 16 keys; afterwards
// key/id[0..count) hold the winners in id order.  On entry the selection
// histograms must be zero (with a barrier since they were cleared).
template <int NT, typename Smem, typename Src>
__device__ __forceinline__ int stream_select(Smem& sm, int64_t n, int k,
                                             Src src) {
  constexpr int kCap = NT * kStreamPer;
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
      constexpr int kH = kStreamPer / 2;
      uint32_t fv[kH];
      int32_t fi[kH];
#pragma unroll
      for (int j = 0; j < kH; ++j) {
        // Unconditional raw loads from a clamped index (n >= 1 whenever
        // fill > 0); keys are formed only after every load is issued.
        const int s = (h * kH + j) * NT + tid;
        int64_t i = pos + (s - count);
        i = i < 0 ? 0 : (i >= n ? (n > 0 ? n - 1 : 0) : i);
        src.load(i, fv[j], fi[j]);
      }
#pragma unroll
      for (int j = 0; j < kH; ++j) {
        const int s = (h * kH + j) * NT + tid;
        if (s >= count && s < count + fill) {
          sm.key[s] = fi[j] >= 0 ? Src::key(fv[j]) : 0u;
          sm.id[s] = fi[j];
        }
      }
    }
    pos += fill;
    __syncthreads();
    count = select_any<NT>(sm, count + fill, k);
  }
  return count;
}

// Element sources (ids ascending in i): load(i, r, id) reads the raw
// 32-bit word and id of element i (always a valid index); key(r) turns the
// word into a selection key -- it already is one when KEYS, else it is a
// float score.
template <bool KEYS>
__device__ __forceinline__ uint32_t word_key(uint32_t r) {
  if constexpr (KEYS) return r;
  else return score_key(__uint_as_float(r));
}
template <bool HAS_IDS, bool KEYS>
struct ScoreSrc {                 // a score row; ids = positions or ids[]
  const uint32_t* row;
  const int32_t* idrow;
  __device__ __forceinline__ void load(int64_t i, uint32_t& r, int32_t& id) const {
    r = row[i];
    id = HAS_IDS ? idrow[i] : (int32_t)i;
  }
  __device__ static __forceinline__ uint32_t key(uint32_t r) {
    return word_key<KEYS>(r);
  }
};

}  // namespace csa2
