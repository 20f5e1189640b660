// Exact block-wide top-k selection over register-held keys (device code).
//
// Order: larger key first, equal keys by lower position (position =
// thread * PER + j, so each thread owns a contiguous run).  Keys are
// order-preserving images of float scores (0 marks an invalid element);
// score_key() canonicalises -0 to +0 so that equal scores have equal keys.
//
// The k-th key is found by narrowing a key interval [lo, hi] that holds it.
// The keys inside are binned by (hi - key) >> shift, with the shift chosen so
// the interval fits NB bins; one wavefront scans the bin counts for the bin
// where the running count from the top reaches the number still needed (and
// clears the bins for the next pass), and the interval becomes exactly that
// bin's key range.  With NB = 2048 a 32-bit range needs at most three passes
// (21, then 10, then 0 bits left).  The search ends with the bin holding
// exactly the number needed (take every key >= lo) or with a one-key
// interval (keys above it, plus the first `need` keys equal to it in
// position order).  One packed prefix sum then yields every selected
// element's output position.  Reductions and scans inside a wavefront use
// DPP row shifts and broadcasts.
#pragma once
#include "common.h"

namespace csa2 {

template <int NT, int NB>
struct SelSmem {
  static_assert((NB & (NB - 1)) == 0 && NB >= 256, "NB is a power of two");
  int32_t hist[NB];
  uint32_t red[4][NT / 64];
  int32_t bstar, cum_before, bcount;
};

// --------------------------------------------------------- wavefront ops --
// Inclusive prefix sum: shifts by 1, 2, 4, 8 inside each 16-lane row, then
// row 15 -> rows 1 and 3 and lane 31 -> rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Wavefront maximum of unsigned keys by the same network (lanes without a
// source keep their own value); the total is read from lane 63.
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL,
                                                      RMASK, 0xf, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max<0x111, 0xf>(v);
  v = dpp_max<0x112, 0xf>(v);
  v = dpp_max<0x114, 0xf>(v);
  v = dpp_max<0x118, 0xf>(v);
  v = dpp_max<0x142, 0xa>(v);
  v = dpp_max<0x143, 0xc>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return ~wave_max_u32(~v);
}

// ------------------------------------------------------------ block ops --
// Block-wide exclusive prefix sum over threads; returns the block total.
template <int NT, int NB>
__device__ __forceinline__ int sel_excl_scan(int x, int& total,
                                             SelSmem<NT, NB>& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) sm.red[0][wv] = (uint32_t)incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int t = (int)sm.red[0][i];
    before += i < wv ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

// Canonical key of a score: NaN and -inf -> 0 (invalid), -0 -> key(+0).
__device__ __forceinline__ uint32_t score_key(float v) {
  if (!(v > -__builtin_inff())) return 0u;
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelResult {
  uint32_t mask;      // selected elements of this thread (bit j)
  int pos;            // selected elements before this thread
  int total;          // selected in the block: min(k, valid keys)
  uint32_t thr;       // every selected key is >= thr, and thr is <= the
                      // smallest selected key (0 when nothing is selected)
};

// Select the top-k (k >= 1) of the NT * PER keys held as key[j] by each
// thread.  The histogram must be all zero on entry; it is all zero again on
// return, and every shared-memory access of the call has completed.
template <int NT, int PER, int NB>
__device__ __forceinline__ SelResult block_select(const uint32_t (&key)[PER],
                                                  int k, SelSmem<NT, NB>& sm) {
  static_assert(PER <= 32, "selection mask is 32 bits");
  static_assert(NT * PER < 65536, "packed counts are 16 bits");
  constexpr int kLogNB = __builtin_ctz(NB);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // Valid count, min and max in one reduction.
  int nval = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (key[j]) { ++nval; mn = min(mn, key[j]); mx = max(mx, key[j]); }
  {
    const int c = __builtin_amdgcn_readlane(wave_incl_scan(nval), 63);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
      sm.red[1][wv] = (uint32_t)c;
      sm.red[2][wv] = mn;
      sm.red[3][wv] = mx;
    }
    __syncthreads();
    nval = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      nval += (int)sm.red[1][i];
      mn = min(mn, sm.red[2][i]);
      mx = max(mx, sm.red[3][i]);
    }
  }

  uint32_t lo = mn, hi = mx;
  int need = k;
  bool take_all = nval <= k;              // select every valid key >= lo
  if (!take_all) {
    for (int it = 0; it < 3 && lo < hi; ++it) {
      const int bits = 32 - __builtin_clz(hi - lo);
      const int shift = bits > kLogNB ? bits - kLogNB : 0;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (key[j] >= lo && key[j] <= hi)
          atomicAdd(&sm.hist[(hi - key[j]) >> shift], 1);
      __syncthreads();
      if (wv == 0) {
        // Wavefront 0 reads the bins (lane L owns bins 32L .. 32L+31, in
        // key order from the top), clears them and finds the crossing.
        constexpr int BPL = NB / 64;
        int cnt[BPL];
        int s = 0;
#pragma unroll
        for (int i = 0; i < BPL; i += 4) {
          int4* p = reinterpret_cast<int4*>(&sm.hist[lane * BPL + i]);
          const int4 v = *p;
          cnt[i] = v.x; cnt[i + 1] = v.y; cnt[i + 2] = v.z; cnt[i + 3] = v.w;
          s += v.x + v.y + v.z + v.w;
          *p = make_int4(0, 0, 0, 0);
        }
        int run = wave_incl_scan(s) - s;
        if (run < need && run + s >= need) {
#pragma unroll
          for (int i = 0; i < BPL; ++i) {
            if (run < need && run + cnt[i] >= need) {
              sm.bstar = lane * BPL + i;
              sm.cum_before = run;
              sm.bcount = cnt[i];
            }
            run += cnt[i];
          }
        }
      }
      __syncthreads();
      const int bs = sm.bstar;
      need -= sm.cum_before;
      const bool exact = sm.bcount == need;
      // The bin's key range, clipped to [lo, hi].
      const uint32_t nhi = hi - ((uint32_t)bs << shift);
      const uint32_t width = (1u << shift) - 1u;
      lo = nhi - lo >= width ? nhi - width : lo;
      hi = nhi;
      if (exact) { take_all = true; break; }
    }
  }
  // Selected: take_all -> key >= lo; else key > hi (= lo) plus the first
  // `need` keys equal to lo.  One packed scan (ties << 16 | greater) gives
  // both counts before this thread.
  int ngt = 0, ntie = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (!key[j]) continue;
    if (take_all) ngt += key[j] >= lo;
    else { ngt += key[j] > hi; ntie += key[j] == lo; }
  }
  int tot;
  const int ex = sel_excl_scan<NT, NB>((ntie << 16) | ngt, tot, sm);
  const int gt_before = ex & 0xFFFF, tie_before = ex >> 16;
  int tie_rank = tie_before;
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    bool s = false;
    if (key[j]) {
      if (take_all) s = key[j] >= lo;
      else if (key[j] > hi) s = true;
      else if (key[j] == lo) { s = tie_rank < need; ++tie_rank; }
    }
    if (s) mask |= 1u << j;
  }
  SelResult res;
  res.mask = mask;
  res.pos = gt_before + (take_all ? 0 : min(tie_before, need));
  const int tot_gt = tot & 0xFFFF, tot_tie = tot >> 16;
  res.total = tot_gt + (take_all ? 0 : min(tot_tie, need));
  res.thr = nval ? lo : 0u;
  return res;
}

}  // namespace csa2
