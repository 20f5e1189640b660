// Exact block-wide top-k selection over register-held keys (device code).
//
// Order: larger key first, equal keys by lower position (position =
// thread * PER + j, so each thread owns a contiguous run).  Keys are
// order-preserving images of float scores (0 marks an invalid element);
// score_key() canonicalises -0 to +0 so that equal scores have equal keys.
//
// The k-th key is found by narrowing a key interval [lo, hi] that holds it.
// Each pass bins the keys inside by (hi - key) >> shift into NB = 256 bins,
// with the shift chosen so the interval fits, in a histogram of its own
// (LDS atomics from every thread); after one barrier every wavefront reads
// the whole histogram (one 16-byte read per lane), finds with one prefix
// scan and a ballot the bin where the running count from the top reaches
// the number still needed, and narrows the interval to exactly that bin's
// key range -- the same decision in every wavefront, so nothing is
// broadcast.  A 32-bit range needs at most four passes (24, 16, 8, then 0
// bits left).  The search ends with the bin holding exactly the number
// needed (take every key >= lo) or with a one-key interval (keys above it,
// plus the first `need` keys equal to it in position order).  One packed
// prefix sum then yields every selected element's output position.
// Reductions and scans inside a wavefront use DPP row shifts and
// broadcasts.
#pragma once
#include "common.h"

namespace csa2 {

template <int NT, int NB>
struct SelSmem {
  static_assert(NB == 256, "the bin scan assumes 4 bins per lane");
  static_assert(NT / 64 >= 4, "one histogram per pass, four passes");
  int32_t hist[NT / 64][NB];      // histogram p serves pass p (all zero
                                  // between calls); the rest is room for
                                  // callers between calls
  uint32_t red[4][NT / 64];
};

// A key range known to hold every valid key, and the number of valid keys
// (lets a selection skip its own min/max reduction).
struct SelRange {
  bool known;
  uint32_t lo, hi;
  int n;
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

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}
// Set bits of m in the lanes below this one, plus `add`.
__device__ __forceinline__ int lanes_below(uint64_t m, int add = 0) {
  return (int)__builtin_amdgcn_mbcnt_hi(
      (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)add));
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

struct SelResult {
  uint32_t mask;      // selected elements of this thread (bit j)
  int pos;            // selected elements before this thread
  int total;          // selected in the block: min(k, valid keys)
  uint32_t thr;       // every selected key is >= thr, thr is <= the
                      // smallest selected key, and at least min(k, valid)
                      // keys are >= thr (0 when no key is valid)
  uint32_t max;       // the largest key (the range's top when known)
  int nval;           // valid (nonzero) keys in the block (the range's
                      // count when known)
};

// Select the top-k (k >= 1) of the NT * PER keys held as key[j] by each
// thread.  On entry the histograms must be zero, with a barrier since the
// previous call returned.  BOUND_ONLY: stop after `passes` passes and return
// only `thr` (a lower bound of the k-th key with at least k keys at or
// above it) and `max`; mask, pos and total are then not set, and the
// histograms are zero again once the caller has passed one more barrier.
// Otherwise they are zero on return and every shared-memory access of the
// call has completed.
template <int NT, int PER, int NB, bool BOUND_ONLY = false>
__device__ __forceinline__ SelResult block_select(
    const uint32_t (&key)[PER], int k, SelSmem<NT, NB>& sm, int passes = 4,
    SelRange range = SelRange{false, 0u, 0u, 0}) {
  static_assert(PER <= 32, "selection mask is 32 bits");
  static_assert(NT * PER < 65536, "packed counts are 16 bits");
  constexpr int kLogNB = 8;
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  int nval;
  uint32_t mn, mx;
  if (range.known) {
    nval = range.n; mn = range.lo; mx = range.hi;
  } else {
    // Valid count, min and max in one reduction.
    nval = 0; mn = 0xFFFFFFFFu; mx = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (key[j]) { ++nval; mn = min(mn, key[j]); mx = max(mx, key[j]); }
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
    for (int i = 0; i < kWaves; ++i) {
      nval += (int)sm.red[1][i];
      mn = min(mn, sm.red[2][i]);
      mx = max(mx, sm.red[3][i]);
    }
  }

  uint32_t lo = mn, hi = mx;
  int need = k;
  bool take_all = nval <= k;              // select every valid key >= lo
  int used = 0;                           // histograms written
  if (!take_all) {
    for (int it = 0; it < passes && lo < hi; ++it) {
      int32_t* H = sm.hist[it];
      const int bits = 32 - __builtin_clz(hi - lo);
      const int shift = bits > kLogNB ? bits - kLogNB : 0;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if ((key[j] >= lo) & (key[j] <= hi))
          atomicAdd(&H[(hi - key[j]) >> shift], 1);
      used = it + 1;
      __syncthreads();
      // Lane L holds bins 4L .. 4L+3 (bins in key order from the top).
      const int4 c = reinterpret_cast<const int4*>(H)[lane];
      const int s = c.x + c.y + c.z + c.w;
      const int run = wave_incl_scan(s) - s;
      // Exactly one lane holds the crossing: `need` >= 1 keys lie in range.
      const bool hit = (run < need) & (run + s >= need);
      const int hl = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(hit));
      int b = 0, before = run, cnt = c.x;
      if (before + c.x < need) {
        before += c.x; b = 1; cnt = c.y;
        if (before + c.y < need) {
          before += c.y; b = 2; cnt = c.z;
          if (before + c.z < need) { before += c.z; b = 3; cnt = c.w; }
        }
      }
      const int bs = __builtin_amdgcn_readlane(4 * lane + b, hl);
      need -= __builtin_amdgcn_readlane(before, hl);
      const bool exact = __builtin_amdgcn_readlane(cnt, hl) == need;
      // The bin's key range, clipped to [lo, hi].
      const uint32_t nhi = hi - ((uint32_t)bs << shift);
      const uint32_t width = (1u << shift) - 1u;
      lo = nhi - lo >= width ? nhi - width : lo;
      hi = nhi;
      if (exact) { take_all = true; break; }
    }
  }
  // Clears the histograms this call wrote (after a barrier that follows
  // every read of them).
  auto clear_used = [&]() {
    for (int i = tid; i < used * NB; i += NT) (&sm.hist[0][0])[i] = 0;
  };
  SelResult res;
  res.thr = nval ? lo : 0u;
  res.max = mx;
  res.nval = nval;
  if constexpr (BOUND_ONLY) {
    res.mask = 0; res.pos = 0; res.total = 0;
    if (used) {
      __syncthreads();
      clear_used();
    }
    return res;
  } else {
    // Selected: take_all -> key >= lo; else key > hi (= lo) plus the first
    // `need` keys equal to lo.  One packed scan (ties << 16 | greater)
    // gives both counts before this thread.
    int ngt = 0, ntie = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (!key[j]) continue;
      if (take_all) ngt += key[j] >= lo;
      else { ngt += key[j] > hi; ntie += key[j] == lo; }
    }
    const int x = (ntie << 16) | ngt;
    const int incl = wave_incl_scan(x);
    if (lane == 63) sm.red[0][wv] = (uint32_t)incl;
    __syncthreads();
    clear_used();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int t = (int)sm.red[0][i];
      before += i < wv ? t : 0;
      tot += t;
    }
    __syncthreads();
    const int ex = before + incl - x;
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
    res.mask = mask;
    res.pos = gt_before + (take_all ? 0 : min(tie_before, need));
    const int tot_gt = tot & 0xFFFF, tot_tie = tot >> 16;
    res.total = tot_gt + (take_all ? 0 : min(tot_tie, need));
    return res;
  }
}

}  // namespace csa2

namespace csa2 {

// ---------------------------------------------------- wavefront select --
struct WaveSelResult {
  uint32_t mask;      // selected elements of this lane (bit j)
  int pos;            // selected elements before this lane
  int total;          // selected in the wavefront: min(k, valid keys)
  uint32_t thr;       // as SelResult::thr: every valid key left out is
                      // <= thr, and thr <= the smallest selected key
  int nval;           // valid (nonzero) keys in the wavefront
};

// Top-k (k >= 1) of the 64 * PER keys held as key[j] by the lanes of one
// wavefront, position = lane * PER + j; larger key first, equal keys to the
// lower position.  The same interval narrowing as block_select, with no
// barrier: H is 256 ints of LDS used by this wavefront alone (zero on entry,
// zero again on return).  The wavefront's own LDS operations take effect in
// issue order, so each pass reads its histogram after its atomics and each
// lane clears the four bins it read before the next pass adds to them.
template <int PER>
__device__ __forceinline__ WaveSelResult wave_select(const uint32_t (&key)[PER],
                                                     int k, int32_t* H) {
  static_assert(PER <= 32, "selection mask is 32 bits");
  static_assert(64 * PER < 65536, "packed counts are 16 bits");
  constexpr int kLogNB = 8;
  const int lane = threadIdx.x & 63;
  int nval = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (key[j]) { ++nval; mn = min(mn, key[j]); mx = max(mx, key[j]); }
  nval = __builtin_amdgcn_readlane(wave_incl_scan(nval), 63);
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t lo = mn, hi = mx;
  int need = k;
  bool take_all = nval <= k;
  if (!take_all) {
    for (int it = 0; it < 4 && lo < hi; ++it) {
      const int bits = 32 - __builtin_clz(hi - lo);
      const int shift = bits > kLogNB ? bits - kLogNB : 0;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if ((key[j] >= lo) & (key[j] <= hi))
          atomicAdd(&H[(hi - key[j]) >> shift], 1);
      int4* hv = reinterpret_cast<int4*>(H) + lane;
      const int4 c = *hv;
      *hv = make_int4(0, 0, 0, 0);
      const int s = c.x + c.y + c.z + c.w;
      const int run = wave_incl_scan(s) - s;
      const bool hit = (run < need) & (run + s >= need);
      const int hl = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(hit));
      int b = 0, before = run, cnt = c.x;
      if (before + c.x < need) {
        before += c.x; b = 1; cnt = c.y;
        if (before + c.y < need) {
          before += c.y; b = 2; cnt = c.z;
          if (before + c.z < need) { before += c.z; b = 3; cnt = c.w; }
        }
      }
      const int bs = __builtin_amdgcn_readlane(4 * lane + b, hl);
      need -= __builtin_amdgcn_readlane(before, hl);
      const bool exact = __builtin_amdgcn_readlane(cnt, hl) == need;
      const uint32_t nhi = hi - ((uint32_t)bs << shift);
      const uint32_t width = (1u << shift) - 1u;
      lo = nhi - lo >= width ? nhi - width : lo;
      hi = nhi;
      if (exact) { take_all = true; break; }
    }
  }
  WaveSelResult res;
  res.thr = nval ? lo : 0u;
  res.nval = nval;
  int ngt = 0, ntie = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (!key[j]) continue;
    if (take_all) ngt += key[j] >= lo;
    else { ngt += key[j] > hi; ntie += key[j] == lo; }
  }
  const int x = (ntie << 16) | ngt;
  const int incl = wave_incl_scan(x);
  const int tot = __builtin_amdgcn_readlane(incl, 63);
  const int ex = incl - x;
  const int gt_before = ex & 0xFFFF, tie_before = ex >> 16;
  int tie_rank = tie_before;
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    bool sel = false;
    if (key[j]) {
      if (take_all) sel = key[j] >= lo;
      else if (key[j] > hi) sel = true;
      else if (key[j] == lo) { sel = tie_rank < need; ++tie_rank; }
    }
    if (sel) mask |= 1u << j;
  }
  res.mask = mask;
  res.pos = gt_before + (take_all ? 0 : min(tie_before, need));
  res.total = (tot & 0xFFFF) + (take_all ? 0 : min(tot >> 16, need));
  return res;
}

// A cut of the wavefront's 64 * PER keys (position = lane * PER + j) that
// keeps at most `cap` of them -- every key >= a threshold t -- and bounds
// the rest: every valid key left out is <= bound (0 when nothing valid is
// left out).  Unlike wave_select it does not find the cap-th key exactly:
// one binning pass over [min, max] and the cut at the lowest bin boundary
// with at most cap keys above it, so the kept count may fall short of cap.
// When the top bin alone holds more than cap keys, the exact wave_select
// decides instead (its threshold is such a bound too).  H as in wave_select.
struct WaveCut {
  uint32_t mask;      // kept elements of this lane (bit j)
  int pos;            // kept elements before this lane
  int total;          // kept in the wavefront
  uint32_t bound;     // every valid key left out is <= bound
};
template <int PER>
__device__ __forceinline__ WaveCut wave_cut(const uint32_t (&key)[PER],
                                            int cap, int32_t* H) {
  constexpr int kLogNB = 8;
  const int lane = threadIdx.x & 63;
  int nval = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (key[j]) { ++nval; mn = min(mn, key[j]); mx = max(mx, key[j]); }
  nval = __builtin_amdgcn_readlane(wave_incl_scan(nval), 63);
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t t = 1u;                      // keep every valid key
  uint32_t bound = 0u;
  if (nval > cap && mx == mn) {
    // One key value held by more than cap keys: the exact selection.
    const WaveSelResult r = wave_select<PER>(key, cap, H);
    WaveCut w;
    w.mask = r.mask;
    w.pos = r.pos;
    w.total = r.total;
    w.bound = r.thr;
    return w;
  }
  if (nval > cap) {
    const int bits = 32 - __builtin_clz(mx - mn);
    const int shift = bits > kLogNB ? bits - kLogNB : 0;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (key[j] >= mn) atomicAdd(&H[(mx - key[j]) >> shift], 1);
    int4* hv = reinterpret_cast<int4*>(H) + lane;
    const int4 c = *hv;
    *hv = make_int4(0, 0, 0, 0);
    // Bins from the top (bin 0 holds mx): the last bin whose running count
    // (through it) is still <= cap.
    const int s = c.x + c.y + c.z + c.w;
    const int run = wave_incl_scan(s) - s;        // keys in earlier bins
    int last = -1;                                // within this lane
    if (run + c.x <= cap) last = 0;
    if (run + c.x + c.y <= cap) last = 1;
    if (run + c.x + c.y + c.z <= cap) last = 2;
    if (run + s <= cap) last = 3;
    const uint64_t any = __builtin_amdgcn_ballot_w64(last >= 0);
    if (any == 0) {
      // The top bin alone holds more than cap keys.
      const WaveSelResult r = wave_select<PER>(key, cap, H);
      WaveCut w;
      w.mask = r.mask;
      w.pos = r.pos;
      w.total = r.total;
      w.bound = r.nval > cap ? r.thr : 0u;
      return w;
    }
    // Running counts only grow, so the qualifying bins are a prefix: the
    // highest qualifying lane holds the cut.
    const int hl = 63 - (int)__builtin_clzll(any);
    const int b = 4 * hl + __builtin_amdgcn_readlane(last, hl);
    // Bin b holds keys in [mx - ((b+1) << shift) + 1, mx - (b << shift)].
    const int64_t low = (int64_t)mx - ((int64_t)(b + 1) << shift) + 1;
    t = low <= (int64_t)mn ? mn : (uint32_t)low;
    bound = t - 1u;                       // keys left out are < t
  }
  int cnt = 0;
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (key[j] != 0u && key[j] >= t) { mask |= 1u << j; ++cnt; }
  const int incl = wave_incl_scan(cnt);
  WaveCut w;
  w.mask = mask;
  w.pos = incl - cnt;
  w.total = __builtin_amdgcn_readlane(incl, 63);
  w.bound = nval > cap && w.total < nval ? bound : 0u;
  return w;
}

}  // namespace csa2
