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
// every top-k element lies in a tile whose maximum is >= M.  One 1024-thread
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
#include "stream_select.h"

namespace csa2 {
namespace {

// A row's selection is a chain of dependent steps (loads, histograms,
// scans), so a workgroup of 16 wavefronts with 16 keys per thread
// finishes it sooner than fewer threads holding more keys each (measured:
// 11.9 us at 1024 threads, 13.1 at 512, 17.7 at 256 for 32 rows of 32,768
// scores).
constexpr int kNT = 1024;                   // threads per row
constexpr int kPer = kStreamPer;            // keys per thread
constexpr int kCap = kNT * kPer;            // 16384 keys per pass
constexpr int kNB = 256;                    // bins per selection pass
constexpr int kTileList = 4000;             // candidate tiles held in LDS

struct RowSmem {
  uint32_t key[kCap];
  int32_t id[kCap];
  int32_t tiles[kTileList];
  SelSmem<kNT, kNB> sel;
  int32_t n_list;                 // listed tiles (-1: the list overflowed)
  uint32_t M;                     // the pruning bound M' (0: no valid score)
  uint32_t M_top;                 // the largest tile maximum
};

// Lanes below this one in the wavefront.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Exclusive prefix of a per-wavefront count over the wavefronts of the
// block (the count is uniform within each wavefront); returns the total.
__device__ __forceinline__ int wave_offset(int wcount, int& total,
                                           SelSmem<kNT, kNB>& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) sm.red[0][wv] = (uint32_t)wcount;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kNT / 64; ++i) {
    const int t = (int)sm.red[0][i];
    before += i < wv ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before;
}

template <bool KEYS>
struct TileSrc {                  // tile maxima; ids = tile numbers
  const uint32_t* trow;
  __device__ __forceinline__ void load(int64_t t, uint32_t& r, int32_t& id) const {
    r = trow[t];
    id = (int32_t)t;
  }
  __device__ static __forceinline__ uint32_t key(uint32_t r) {
    return word_key<KEYS>(r);
  }
};

struct RowArgs {
  const void* scores;       // float scores or keys; row stride ld
  const void* tmax;         // nullable, same form; row stride ceil(n_cols/32)
  int64_t ld;               // keys without ids: a multiple of 32
  int64_t n_cols;           // row length (<= ld); ids row stride
  const int32_t* n_valid;   // nullable
  int valid_div;            // row length ceil(n_valid[b] / valid_div)
  const int32_t* ids;       // nullable
  int k;
  int block;
  const int32_t* limit;     // nullable
  int32_t* out;             // [B][k * block]
};

// Write chosen id `id` as output entry p (expanded by `block`, clipped).
__device__ __forceinline__ void put(const RowArgs& a, int64_t ob, int64_t lim,
                                    int p, int64_t id) {
  for (int t = 0; t < a.block; ++t) {
    const int64_t q = id * a.block + t;
    a.out[ob + (int64_t)p * a.block + t] = q < lim ? (int32_t)q : -1;
  }
}

// Final selection over the `count` candidates in sm.key/sm.id (ids in
// order), written straight to the output at the positions the selection
// gives.  Returns the number chosen.
template <int PER>
__device__ __forceinline__ int select_out(RowSmem& sm, int count,
                                          const RowArgs& a, int64_t ob,
                                          int64_t lim, SelRange range) {
  const int tid = threadIdx.x;
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {       // unconditional reads, then masks
    const int pos = tid * PER + j;
    const uint32_t kv = sm.key[pos];
    key[j] = pos < count ? kv : 0u;
  }
  const SelResult r = block_select<kNT, PER, kNB>(key, a.k, sm.sel, 4, range);
  int32_t idv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) idv[j] = sm.id[tid * PER + j];
  int p = r.pos;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (r.mask & (1u << j)) put(a, ob, lim, p++, idv[j]);
  return r.total;
}

// Pruning steps (1) and (2) of the file comment: M', a lower bound of the
// k-th largest tile maximum with at least k tile maxima at or above it
// (two binning passes: a bound is enough, the candidates only grow by the
// few tiles that share M's bin), and the list of tiles whose maximum is
// >= M', in order, in sm.tiles.  Both end in sm.n_list / sm.M (n_list is
// -1 when the list does not fit).  TP tile maxima per thread (thread t owns
// tiles TP*t .. TP*t+TP-1), read coalesced and staged as keys in sm.key.
template <int TP, bool KEYS>
__device__ __forceinline__ void block_tile_list(RowSmem& sm,
                                                const uint32_t* trow,
                                                int n_t, int k) {
  const int tid = threadIdx.x;
  {
    uint32_t tv[TP];
#pragma unroll
    for (int r = 0; r < TP; ++r) {
      const int t = r * kNT + tid;
      tv[r] = trow[t < n_t ? t : n_t - 1];
    }
#pragma unroll
    for (int r = 0; r < TP; ++r) {
      const int t = r * kNT + tid;
      sm.key[t] = t < n_t ? word_key<KEYS>(tv[r]) : 0u;
    }
  }
  __syncthreads();
  uint32_t tk[TP];
#pragma unroll
  for (int j = 0; j < TP; ++j) tk[j] = sm.key[tid * TP + j];
  const SelResult r = block_select<kNT, TP, kNB, true>(tk, k, sm.sel, 2);
  const uint32_t M = r.thr;
  uint32_t fl = 0;
#pragma unroll
  for (int j = 0; j < TP; ++j)
    if ((tk[j] >= M) & (M != 0)) fl |= 1u << j;
  int n_list;
  int p = sel_excl_scan<kNT, kNB>(__popc(fl), n_list, sm.sel);
  if (n_list <= kTileList) {
#pragma unroll
    for (int j = 0; j < TP; ++j)
      if (fl & (1u << j)) sm.tiles[p++] = tid * TP + j;
  }
  if (tid == 0) {
    sm.n_list = n_list <= kTileList ? n_list : -1;
    sm.M = M;
    sm.M_top = r.max;
  }
}

// Leaves sm.n_list / sm.M / sm.tiles set and visible to every thread.
template <int TP, bool KEYS>
__device__ __forceinline__ void tile_list(RowSmem& sm, const uint32_t* trow,
                                          int n_t, int k) {
  if constexpr (TP < kPer) {
    if (n_t > kNT * TP) return tile_list<TP * 2, KEYS>(sm, trow, n_t, k);
  }
  block_tile_list<TP, KEYS>(sm, trow, n_t, k);
  __syncthreads();
}

// Pruning step (3): the elements >= M' of the listed tiles, into
// sm.key/sm.id in id order; returns their number, or -1 when they do not
// fit.  A wavefront covers 8 listed tiles per step: lanes 8j..8j+7 take tile
// j, four consecutive elements each, so a lane's elements, then the lanes,
// then the steps, then the wavefronts run in id order.  S steps per
// wavefront and round (S chosen so one round usually covers the list).
// Places are counted by ballots: an element's place is the kept elements of
// lower lanes (the four per-element ballots' counts below this lane) plus
// this lane's earlier ones.
template <int S, bool HAS_IDS, bool KEYS>
__device__ __forceinline__ int gather_candidates(
    RowSmem& sm, int n_list, uint32_t M, int64_t len,
    const ScoreSrc<HAS_IDS, KEYS>& src) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int len32 = (int)len;                 // < 2^20 here (n_t <= 16384)
  // Key rows without ids are padded to whole tiles (the row stride is a
  // multiple of 32 entries), so each lane's four entries are one aligned
  // 16-byte load; otherwise four single loads, moved back at the row's end.
  constexpr bool kVec = KEYS && !HAS_IDS;
  constexpr int kChunk = kNT / 64 * 8 * S;    // listed tiles per round
  const int sub = 4 * (lane & 7);             // first element in the tile
  int n_c = 0;
  for (int c0 = 0; c0 < n_list; c0 += kChunk) {
    int pos[S];
    uint32_t w[S][4];
    int32_t id[S][4];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int li = c0 + (wv * S + s) * 8 + (lane >> 3);
      if constexpr (kVec) {
        // An unlisted slot reads listed tile 0 and is masked out by pos.
        const int t = sm.tiles[li < n_list ? li : 0];
        pos[s] = li < n_list ? t * 32 + sub : len32;
        const uint4 v =
            *reinterpret_cast<const uint4*>(src.row + (t * 32 + sub));
        w[s][0] = v.x; w[s][1] = v.y; w[s][2] = v.z; w[s][3] = v.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) id[s][e] = pos[s] + e;   // the position
      } else {
        pos[s] = li < n_list ? sm.tiles[li] * 32 + sub : len32;  // len: none
      }
    }
    if constexpr (!kVec) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        // Four loads from one address: at the row's end the run is moved
        // back to stay inside it (len >= 33 here) and shifted into place.
        const int pc = pos[s] < len32 - 4 ? pos[s] : len32 - 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) src.load(pc + e, w[s][e], id[s][e]);
        const int d = pos[s] - pc;                   // 0 except at the end
        if (d > 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int f = e + d < 4 ? e + d : 3;
            w[s][e] = f == 1 ? w[s][1] : f == 2 ? w[s][2] : w[s][3];
            id[s][e] = f == 1 ? id[s][1] : f == 2 ? id[s][2] : id[s][3];
          }
        }
      }
    }
    uint32_t keep[S];                                // 4 bits per step
    int lcount = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      keep[s] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // Past the row's end (padding, or an unlisted slot) nothing is kept.
        const bool kp = (pos[s] + e < len32) & (id[s][e] >= 0) &
                        (word_key<KEYS>(w[s][e]) >= M);
        keep[s] |= (kp ? 1u : 0u) << e;
      }
      lcount += __popc(keep[s]);
    }
    const int wcount = __builtin_amdgcn_readlane(wave_incl_scan(lcount), 63);
    int total;
    int run = n_c + wave_offset(wcount, total, sm.sel);
    if (n_c + total <= kCap) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        uint64_t m[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = wave_ballot((keep[s] >> e) & 1u);
        int q = run;
#pragma unroll
        for (int e = 0; e < 4; ++e) q = lanes_below(m[e], q);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((keep[s] >> e) & 1u) {
            sm.key[q] = word_key<KEYS>(w[s][e]);
            sm.id[q] = id[s][e];
            ++q;
          }
        run += __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) +
               __popcll(m[3]);
      }
    }
    n_c += total;
  }
  __syncthreads();
  return n_c <= kCap ? n_c : -1;
}

template <bool HAS_IDS, bool KEYS>
__device__ __forceinline__ int gather_dispatch(
    RowSmem& sm, int n_list, uint32_t M, int64_t len,
    const ScoreSrc<HAS_IDS, KEYS>& src) {
  if (n_list <= kNT / 64 * 8 * 2)
    return gather_candidates<2, HAS_IDS, KEYS>(sm, n_list, M, len, src);
  if (n_list <= kNT / 64 * 8 * 4)
    return gather_candidates<4, HAS_IDS, KEYS>(sm, n_list, M, len, src);
  // Longer lists take more rounds of 8 steps (16 steps per round would
  // need more registers than 16 wavefronts per workgroup allow).
  return gather_candidates<8, HAS_IDS, KEYS>(sm, n_list, M, len, src);
}

// One row b of a selection (the workgroup's whole work).
template <bool HAS_IDS, bool KEYS>
__device__ __forceinline__ void row_select_row(const RowArgs& a, int b) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  RowSmem& sm = *reinterpret_cast<RowSmem*>(smem_raw);
  const int tid = threadIdx.x;
  for (int i = tid; i < kNT / 64 * kNB; i += kNT) (&sm.sel.hist[0][0])[i] = 0;
  int64_t len = a.n_cols;
  if (a.n_valid) {
    const int32_t v = a.n_valid[b];
    const int64_t nv = v <= 0 ? 0 : ((int64_t)v + a.valid_div - 1) / a.valid_div;
    len = nv < len ? nv : len;
  }
  const ScoreSrc<HAS_IDS, KEYS> from_scores{
      static_cast<const uint32_t*>(a.scores) + (int64_t)b * a.ld,
      HAS_IDS ? a.ids + (int64_t)b * a.n_cols : nullptr};
  const int64_t ob = (int64_t)b * a.k * a.block;
  const int64_t lim = a.limit ? (int64_t)a.limit[b] : INT64_MAX;
  const int64_t n_t = (len + 31) >> 5;
  int count = -1;
  if (a.tmax != nullptr && n_t > a.k && n_t <= (int64_t)kNT * kPer) {
    const uint32_t* trow = static_cast<const uint32_t*>(a.tmax) +
                           (int64_t)b * ((a.n_cols + 31) >> 5);
    tile_list<2, KEYS>(sm, trow, (int)n_t, a.k);
    const int n_list = sm.n_list;
    const uint32_t M = sm.M;
    int n_c = -1;
    if (M == 0) n_c = 0;                      // no valid score at all
    else if (n_list >= 0)
      n_c = gather_dispatch<HAS_IDS, KEYS>(sm, n_list, M, len, from_scores);
    if (n_c >= 0) {
      // Every candidate lies in [M', largest tile maximum].
      const SelRange range{true, M, sm.M_top, n_c};
      if (n_c <= kNT * 2) count = select_out<2>(sm, n_c, a, ob, lim, range);
      else if (n_c <= kNT * 8) count = select_out<8>(sm, n_c, a, ob, lim, range);
      else count = select_out<kPer>(sm, n_c, a, ob, lim, range);
    }
  }
  if (count < 0) {
    // Whole-row streaming (short rows, or candidates that overflow).
    __syncthreads();
    count = stream_select<kNT>(sm, len, a.k, from_scores);
    for (int p = tid; p < count; p += kNT) put(a, ob, lim, p, sm.id[p]);
  }
  for (int64_t p = (int64_t)count * a.block + tid; p < (int64_t)a.k * a.block;
       p += kNT)
    a.out[ob + p] = -1;
}

template <bool HAS_IDS, bool KEYS>
__global__ __launch_bounds__(kNT) void row_select_kernel(RowArgs a) {
  row_select_row<HAS_IDS, KEYS>(a, blockIdx.x);
}

// Two independent key selections in one launch, side by side: workgroups
// 0 .. B0-1 take the rows of a0, the rest those of a1.
__global__ __launch_bounds__(kNT) void row_select_pair_kernel(RowArgs a0,
                                                              RowArgs a1,
                                                              int B0) {
  if ((int)blockIdx.x < B0) row_select_row<false, true>(a0, blockIdx.x);
  else row_select_row<false, true>(a1, (int)blockIdx.x - B0);
}

// ------------------------------------------------- two-stage selection --
// Long rows with few of them (too little parallelism for one workgroup per
// row) split into chunks of kChunk entries.  Stage 1 (a workgroup per
// chunk) keeps each chunk's top kl (key, id) pairs in id order and a bound
// on what it left out: every valid key not kept is <= the selection's
// threshold (0 when the chunk kept all its valid keys).  Stage 2 (a
// workgroup per row) selects the row's top k from the union of its chunks'
// pairs: with L the largest bound, when at least k pairs have keys above L
// their top k is the row's (anything left out is <= L), and with fewer the
// union is the whole answer only when L = 0; otherwise the row streams
// through the exact selection instead.
constexpr int kChunkNT = 256;
constexpr int kChunk = kChunkNT * kPer;     // 4096 entries per chunk
constexpr int kSplitCap = kNT * 8;          // union pairs per row (8,192)

struct SplitArgs {
  RowArgs a;
  int G;                    // chunks per row
  int kl;                   // pairs kept per chunk
  uint2* cand;              // [B][G][kl] (key, id), id order
  uint32_t* bound;          // [B][G]
};

struct ChunkSmem {
  uint32_t key[kChunk];
  int32_t id[kChunk];
  SelSmem<kChunkNT, kNB> sel;
};

__device__ __forceinline__ int64_t row_len(const RowArgs& a, int b) {
  int64_t len = a.n_cols;
  if (a.n_valid) {
    const int32_t v = a.n_valid[b];
    const int64_t nv = v <= 0 ? 0 : ((int64_t)v + a.valid_div - 1) / a.valid_div;
    len = nv < len ? nv : len;
  }
  return len;
}

// Stage 1: chunk blockIdx.x of row blockIdx.y.  Entries are read coalesced
// into LDS (an entry past the row or with a negative id has key 0), then
// thread t takes entries 16t .. 16t+15 of the chunk, so the selection's
// position order is id order.
template <bool HAS_IDS, bool KEYS>
__global__ __launch_bounds__(kChunkNT) void chunk_select_kernel(SplitArgs sa) {
  __shared__ ChunkSmem sm;
  const RowArgs& a = sa.a;
  const int b = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < kChunkNT / 64 * kNB; i += kChunkNT)
    (&sm.sel.hist[0][0])[i] = 0;
  const int64_t len = row_len(a, b);
  const int64_t base = (int64_t)g * kChunk;
  const uint32_t* row = static_cast<const uint32_t*>(a.scores) + (int64_t)b * a.ld;
  const int32_t* idr = HAS_IDS ? a.ids + (int64_t)b * a.n_cols : nullptr;
  uint32_t w[kPer];
  int32_t iv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = base + j * kChunkNT + tid;
    const int64_t ic = i < len ? i : (len > 0 ? len - 1 : 0);
    w[j] = len > 0 ? row[ic] : 0u;
    iv[j] = HAS_IDS ? (len > 0 ? idr[ic] : -1) : (int32_t)i;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = base + j * kChunkNT + tid;
    const bool ok = i < len && iv[j] >= 0;
    sm.key[j * kChunkNT + tid] = ok ? word_key<KEYS>(w[j]) : 0u;
    sm.id[j * kChunkNT + tid] = iv[j];
  }
  __syncthreads();
  uint32_t kk[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) kk[j] = sm.key[tid * kPer + j];
  const SelResult r = block_select<kChunkNT, kPer, kNB>(kk, sa.kl, sm.sel);
  const int64_t grp = (int64_t)b * sa.G + g;
  uint2* co = sa.cand + grp * sa.kl;
  int p = r.pos;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (r.mask & (1u << j))
      co[p++] = make_uint2(kk[j], (uint32_t)sm.id[tid * kPer + j]);
  for (int q = r.total + tid; q < sa.kl; q += kChunkNT)
    co[q] = make_uint2(0u, 0xFFFFFFFFu);
  if (tid == 0) sa.bound[grp] = r.nval > sa.kl ? r.thr : 0u;
}

// Stage 2 for row blockIdx.x: PER union pairs per thread (thread t holds
// pairs PER*t .. PER*t+PER-1, in id order).
template <int PER, bool HAS_IDS, bool KEYS>
__device__ __forceinline__ void union_row(const SplitArgs& sa, int b) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  RowSmem& sm = *reinterpret_cast<RowSmem*>(smem_raw);
  const RowArgs& a = sa.a;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < kNT / 64 * kNB; i += kNT) (&sm.sel.hist[0][0])[i] = 0;
  const int U = sa.G * sa.kl;
  const uint2* cr = sa.cand + (int64_t)b * U;
  uint32_t kk[PER];
  int32_t ci[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    const uint2 v = cr[i < U ? i : U - 1];
    kk[j] = i < U ? v.x : 0u;
    ci[j] = (int32_t)v.y;
  }
  uint32_t lb = 0u;
  for (int i = tid; i < sa.G; i += kNT)
    lb = max(lb, sa.bound[(int64_t)b * sa.G + i]);
  lb = wave_max_u32(lb);
  if (lane == 0) sm.sel.red[0][wv] = lb;
  __syncthreads();
  uint32_t L = 0u;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) L = max(L, sm.sel.red[0][w]);
  __syncthreads();                  // red[] is the selection's scratch too
#pragma unroll
  for (int j = 0; j < PER; ++j) kk[j] = kk[j] > L ? kk[j] : 0u;
  const SelResult r = block_select<kNT, PER, kNB>(kk, a.k, sm.sel);
  const int64_t ob = (int64_t)b * a.k * a.block;
  const int64_t lim = a.limit ? (int64_t)a.limit[b] : INT64_MAX;
  int count;
  if (r.nval >= a.k || L == 0u) {
    int p = r.pos;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (r.mask & (1u << j)) put(a, ob, lim, p++, ci[j]);
    count = r.total;
  } else {
    // Not provably exact: the whole row through the streaming selection.
    const ScoreSrc<HAS_IDS, KEYS> from_scores{
        static_cast<const uint32_t*>(a.scores) + (int64_t)b * a.ld,
        HAS_IDS ? a.ids + (int64_t)b * a.n_cols : nullptr};
    __syncthreads();
    count = stream_select<kNT>(sm, row_len(a, b), a.k, from_scores);
    for (int p = tid; p < count; p += kNT) put(a, ob, lim, p, sm.id[p]);
  }
  for (int64_t p = (int64_t)count * a.block + tid; p < (int64_t)a.k * a.block;
       p += kNT)
    a.out[ob + p] = -1;
}

template <int PER, bool HAS_IDS, bool KEYS>
__global__ __launch_bounds__(kNT) void union_select_kernel(SplitArgs sa) {
  union_row<PER, HAS_IDS, KEYS>(sa, blockIdx.x);
}

// Tile maxima of a plain score array.  Entries at or past the row's length
// (n_valid[b] when given) and entries with a negative id count as -inf, so a
// tile maximum is always the maximum of scores the selection may choose: a
// stale value past the length must not lift a tile above the pruning bound.
// One thread per tile.
__global__ void tilemax_kernel(const float* __restrict__ scores, int64_t ld,
                               const int32_t* __restrict__ ids,
                               const int32_t* __restrict__ n_valid, int B,
                               float* __restrict__ tmax) {
  const int64_t nt = (ld + 31) >> 5;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nt * B) return;
  const int64_t b = t / nt, tt = t % nt;
  int64_t len = ld;
  if (n_valid) {
    const int32_t v = n_valid[b];
    len = v <= 0 ? 0 : ((int64_t)v < ld ? (int64_t)v : ld);
  }
  float mx = -__builtin_inff();
  for (int j = 0; j < 32; ++j) {
    const int64_t i = tt * 32 + j;
    if (i >= len) break;
    const float v = scores[b * ld + i];
    if ((!ids || ids[b * ld + i] >= 0) && v > mx) mx = v;
  }
  tmax[t] = mx;
}

}  // namespace

SplitPlan split_plan(int B, int64_t n_cols, int k) {
  SplitPlan sp;
  // Worth it when one workgroup per row leaves most of the GPU idle and
  // the row spans several chunks.
  if (B < 1 || B > 128 || k < 1 || k > 2048 || n_cols < 2 * kChunk)
    return sp;
  const int64_t G = (n_cols + kChunk - 1) / kChunk;
  // A chunk expects mu = k * kChunk / n_cols of the row's winners; it keeps
  // 2 mu + 24 (on independent scores more than that is many standard
  // deviations away: for mu = 2, P(X > 28) < 1e-15), at most the chunk.
  int64_t kl = 2 * (((int64_t)k * kChunk + n_cols - 1) / n_cols) + 24;
  kl = std::min<int64_t>(kl, kChunk);
  if (G * kl > kSplitCap) return sp;
  sp.ok = true;
  sp.G = (int)G;
  sp.kl = (int)kl;
  return sp;
}

size_t split_workspace(int B, int64_t n_cols, int k) {
  const SplitPlan sp = split_plan(B, n_cols, k);
  if (!sp.ok) return 0;
  return ((((size_t)B * sp.G * sp.kl * 8) + 255) & ~size_t(255)) +
         ((((size_t)B * sp.G * 4) + 255) & ~size_t(255));
}

size_t topk_workspace(int B, int64_t ld, int k) {
  const size_t tm = ld <= kCap ? 0
      : (((size_t)B * ((ld + 31) >> 5) * 4) + 255) & ~size_t(255);
  return tm + split_workspace(B, ld, k);
}

template <int PER, bool HAS_IDS, bool KEYS>
hipError_t launch_union(const SplitArgs& sa, int B, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit(
      reinterpret_cast<const void*>(union_select_kernel<PER, HAS_IDS, KEYS>),
      (int)sizeof(RowSmem), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((union_select_kernel<PER, HAS_IDS, KEYS>), dim3((unsigned)B),
                     dim3(kNT), sizeof(RowSmem), s, sa);
  return hipGetLastError();
}

template <bool HAS_IDS, bool KEYS>
hipError_t launch_split(const RowArgs& a, const SplitPlan& sp, void* ws,
                        int B, hipStream_t s) {
  SplitArgs sa;
  sa.a = a;
  sa.G = sp.G;
  sa.kl = sp.kl;
  sa.cand = static_cast<uint2*>(ws);
  sa.bound = reinterpret_cast<uint32_t*>(
      static_cast<uint8_t*>(ws) +
      ((((size_t)B * sp.G * sp.kl * 8) + 255) & ~size_t(255)));
  hipLaunchKernelGGL((chunk_select_kernel<HAS_IDS, KEYS>),
                     dim3((unsigned)sp.G, (unsigned)B), dim3(kChunkNT), 0, s,
                     sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int U = sp.G * sp.kl;
  if (U <= kNT * 2) return launch_union<2, HAS_IDS, KEYS>(sa, B, s);
  if (U <= kNT * 4) return launch_union<4, HAS_IDS, KEYS>(sa, B, s);
  return launch_union<8, HAS_IDS, KEYS>(sa, B, s);
}

template <bool HAS_IDS, bool KEYS>
hipError_t launch_rows(const RowArgs& a, int B, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit(
      reinterpret_cast<const void*>(row_select_kernel<HAS_IDS, KEYS>),
      (int)sizeof(RowSmem), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((row_select_kernel<HAS_IDS, KEYS>), dim3((unsigned)B),
                     dim3(kNT), sizeof(RowSmem), s, a);
  return hipGetLastError();
}

RowArgs row_args(const void* scores, const void* tmax, int64_t ld,
                 int64_t n_cols, const int32_t* n_valid, const int32_t* ids,
                 int k, int block, const int32_t* limit, int32_t* out) {
  RowArgs a{};
  a.scores = scores;
  a.tmax = tmax;
  a.ld = ld;
  a.n_cols = n_cols;
  a.n_valid = n_valid;
  a.valid_div = 1;
  a.ids = ids;
  a.k = k;
  a.block = block;
  a.limit = limit;
  a.out = out;
  return a;
}

hipError_t launch_row_select(const void* scores, const void* tmax, bool keys,
                             int64_t ld, int64_t n_cols,
                             const int32_t* n_valid, const int32_t* ids, int B,
                             int k, int block, const int32_t* limit,
                             int32_t* out, hipStream_t s, int valid_div,
                             void* split_ws) {
  if (B == 0) return hipSuccess;
  if (n_cols > ld || (keys && !ids && (ld & 31)) || valid_div < 1)
    return hipErrorInvalidValue;
  RowArgs a = row_args(scores, tmax, ld, n_cols, n_valid, ids, k, block,
                       limit, out);
  a.valid_div = valid_div;
  const SplitPlan sp = split_plan(B, n_cols, k);
  if (split_ws && sp.ok) {
    if (ids) return keys ? launch_split<true, true>(a, sp, split_ws, B, s)
                         : launch_split<true, false>(a, sp, split_ws, B, s);
    return keys ? launch_split<false, true>(a, sp, split_ws, B, s)
                : launch_split<false, false>(a, sp, split_ws, B, s);
  }
  if (ids) return keys ? launch_rows<true, true>(a, B, s)
                       : launch_rows<true, false>(a, B, s);
  return keys ? launch_rows<false, true>(a, B, s)
              : launch_rows<false, false>(a, B, s);
}

hipError_t launch_row_select_pair(const KeyRows& r0, const KeyRows& r1, int B,
                                  hipStream_t s) {
  if (B == 0) return hipSuccess;
  for (const KeyRows* r : {&r0, &r1})
    if (r->n_cols > r->ld || (r->ld & 31)) return hipErrorInvalidValue;
  const RowArgs a0 = row_args(r0.keys, r0.tmax, r0.ld, r0.n_cols, r0.n_valid,
                              nullptr, r0.k, r0.block, r0.limit, r0.out);
  const RowArgs a1 = row_args(r1.keys, r1.tmax, r1.ld, r1.n_cols, r1.n_valid,
                              nullptr, r1.k, r1.block, r1.limit, r1.out);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit(
      reinterpret_cast<const void*>(row_select_pair_kernel),
      (int)sizeof(RowSmem), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_select_pair_kernel, dim3((unsigned)(2 * B)),
                     dim3(kNT), sizeof(RowSmem), s, a0, a1, B);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid,
                       const int32_t* ids, int B, int k, int block,
                       const int32_t* limit, int32_t* out, void* ws,
                       hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (split_plan(B, ld, k).ok)        // the two-stage selection
    return launch_row_select(scores, nullptr, false, ld, ld, n_valid, ids, B,
                             k, block, limit, out, s, 1, ws);
  float* tmax = nullptr;
  if (ld > kCap) {
    tmax = static_cast<float*>(ws);
    const int64_t n = (int64_t)B * ((ld + 31) >> 5);
    hipLaunchKernelGGL(tilemax_kernel, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, scores, ld, ids, n_valid, B, tmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_row_select(scores, tmax, false, ld, ld, n_valid, ids, B, k,
                           block, limit, out, s);
}

}  // namespace csa2
