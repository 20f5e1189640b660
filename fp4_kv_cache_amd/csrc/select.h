// Exact block-wide top-k selection over register-held keys (device code).
//
// Order: larger key first, equal keys by lower position (position =
// thread * PER + j, so each thread owns a contiguous run).  Keys are
// order-preserving images of float scores (0 marks an invalid element);
// the caller canonicalises -0 to +0 so that equal scores have equal keys.
//
// The k-th key is found by narrowing a key interval [lo, hi] that holds it.
// The candidates inside are binned by (hi - key) >> shift, with the shift
// chosen so the range fits NB bins (monotone, one subtract and one shift per
// element); a block scan locates the bin where the running count from the top
// reaches the number still needed, and the interval becomes that bin's actual
// [min, max].  Each pass shrinks a 32-bit key range at least NB/2-fold, so a
// few passes suffice; the search ends with the bin holding exactly the number
// needed, or with all candidates equal (then the lowest positions win).
#pragma once
#include "common.h"

namespace csa2 {

template <int NT, int NB>
struct SelSmem {
  static_assert((NB & (NB - 1)) == 0, "NB is a power of two");
  int32_t hist[NB];
  int32_t red[NT / 64];
  uint32_t kred[2][NT / 64];
  int32_t bstar, cum_before;
};

// Wavefront inclusive prefix sum with DPP: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then row 15 -> rows 1 and 3 and lane 31 -> rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Wavefront min and max of unsigned keys (result in every lane).
__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
}

// Block-wide exclusive prefix sum over threads; returns the block total.
template <int NT, int NB>
__device__ __forceinline__ int sel_excl_scan(int x, int& total,
                                             SelSmem<NT, NB>& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) sm.red[wv] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int t = sm.red[i];
    before += i < wv ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

template <int NT, int NB>
__device__ __forceinline__ void sel_minmax(uint32_t& mn, uint32_t& mx,
                                           SelSmem<NT, NB>& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  wave_minmax(mn, mx);
  if (lane == 0) { sm.kred[0][wv] = mn; sm.kred[1][wv] = mx; }
  __syncthreads();
  mn = sm.kred[0][0];
  mx = sm.kred[1][0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) {
    mn = min(mn, sm.kred[0][i]);
    mx = max(mx, sm.kred[1][i]);
  }
  __syncthreads();
}

__device__ __forceinline__ int sel_bin(uint32_t key, uint32_t hi, int shift) {
  return (int)((hi - key) >> shift);
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
  int n_valid;        // block total of valid elements
};

// Select the top-k of the NT * PER keys held as key[j] by each thread.
template <int NT, int PER, int NB>
__device__ __forceinline__ SelResult block_select(const uint32_t (&key)[PER], int k,
                                  SelSmem<NT, NB>& sm) {
  static_assert(PER <= 32, "selection mask is 32 bits");
  const int tid = threadIdx.x;
  int nval = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (key[j]) { ++nval; mn = min(mn, key[j]); mx = max(mx, key[j]); }
  SelResult res;
  sel_excl_scan<NT, NB>(nval, res.n_valid, sm);
  sel_minmax<NT, NB>(mn, mx, sm);

  uint32_t lo = mn, hi = mx;
  int need = k;
  bool take_all = true;                   // select every key >= lo
  if (res.n_valid > k) {
    take_all = false;                     // else: key > hi, plus the first
    for (int it = 0; it < 16; ++it) {     // `need` keys equal to lo
      if (lo == hi) break;
      // smallest shift with (hi - lo) >> shift < NB
      constexpr int kLogNB = __builtin_ctz(NB);
      const int bits = 32 - __builtin_clz(hi - lo);
      const int shift = bits > kLogNB ? bits - kLogNB : 0;
      for (int i = tid; i < NB; i += NT) sm.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (key[j] >= lo && key[j] <= hi)
          atomicAdd(&sm.hist[sel_bin(key[j], hi, shift)], 1);
      __syncthreads();
      constexpr int BPT = NB / NT > 0 ? NB / NT : 1;   // bins per thread
      int hs[BPT];
      int my = 0;
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        const int bin = tid * BPT + i;
        hs[i] = bin < NB ? sm.hist[bin] : 0;
        my += hs[i];
      }
      int tot;
      int run = sel_excl_scan<NT, NB>(my, tot, sm);
      if (run < need && run + my >= need) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          if (run < need && run + hs[i] >= need) {
            sm.bstar = tid * BPT + i;
            sm.cum_before = run;
          }
          run += hs[i];
        }
      }
      __syncthreads();
      const int bs = sm.bstar;
      const int cnt = sm.hist[bs];
      need -= sm.cum_before;
      uint32_t bmn = 0xFFFFFFFFu, bmx = 0u;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (key[j] >= lo && key[j] <= hi && sel_bin(key[j], hi, shift) == bs) {
          bmn = min(bmn, key[j]);
          bmx = max(bmx, key[j]);
        }
      sel_minmax<NT, NB>(bmn, bmx, sm);
      lo = bmn;
      hi = bmx;
      if (cnt == need) { take_all = true; break; }
    }
  }
  // Ranks among the keys equal to lo (in position order).
  int ntie = 0;
  if (!take_all) {
#pragma unroll
    for (int j = 0; j < PER; ++j) ntie += key[j] == lo ? 1 : 0;
  }
  int tie_total;
  int tie_rank = sel_excl_scan<NT, NB>(ntie, tie_total, sm);
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    bool s;
    if (!key[j]) s = false;
    else if (take_all) s = key[j] >= lo;
    else if (key[j] > hi) s = true;
    else if (key[j] == lo) { s = tie_rank < need; ++tie_rank; }
    else s = false;
    if (s) mask |= 1u << j;
  }
  res.mask = mask;
  return res;
}

}  // namespace csa2
