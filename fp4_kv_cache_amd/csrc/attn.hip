// Gather + dequant of the selected FP4 main-KV entries and the E4M3 window,
// and 64-head shared-latent attention over them (one decode query per
// sequence).
//
// Sources: "DeepSeek-V4: Towards Highly Efficient Million-Token Context
// Intelligence" (baisen.site), CSA step 3 (o_{t,i} = CoreAttn(q_{t,i}, C, C),
// softmax(q K^T / sqrt(c)) V with every selected entry serving as key and
// value) and the sliding-window paragraph (the window rows are concatenated
// with the selected entries); "DeepSeek-V4.1-Flash: Pushing the Limits of KV
// Cache Compression" (mer.run) section 4.1 attention line and section 5
// (the cache is dequantised before attention; FP4 is storage only);
// "DeepSeek-V4.1-Flash, 2. Architecture" section 2.4.4.
//
// gfx950 mapping.  A workgroup of 8 wavefronts owns one sequence and a
// contiguous range of key slots (slots 0..k-1 are the chosen main entries,
// k..k+127 the window rows).  Wavefronts 0..3 do the products (wavefront w:
// heads 16w..16w+15, queries and accumulators resident in registers);
// wavefronts 4..7 gather and dequantise the next tile meanwhile, one of each
// kind per SIMD, meeting at one barrier per tile.  Key tiles of 32 slots
// are gathered straight from HBM (one 256-byte code row per wavefront
// instruction), dequantised exactly to fp16 and written to LDS once,
// key-major (rows padded by 32 bytes).  Both products run on
// v_mfma_f32_16x16x32_f16: S^T = K Q^T reads 16-byte key rows, and
// O^T = V^T P^T reads the same tile through gfx950's transposing LDS read
// (ds_read_b64_tr_b16), so the keys need no second, slot-grouped copy.
//
// Why fp16: an E2M1 value times an E4M3 scale has at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in fp16, and the scale
// multiply is one packed fp16 multiply after the FP4->fp16 convert (the
// hardware convert applies only the exponent of its scale operand).  E4M3
// window values are exact in fp16 too.  The bf16 queries are converted to
// fp16 once, each head prescaled by a power of two (exact; see the kernel),
// and probabilities in fp16 keep 11 significant bits.
//
// The S^T output layout equals the P^T operand layout, so probabilities never
// leave registers.  Softmax is online in float32 with the exp2 reference
// point moved only when the tile maximum rises by more than 2^8 (exact
// algebra, fewer rescales).  LDS is double buffered: the gather of tile t+1
// is in flight while tile t runs on the matrix cores.  With several
// workgroups per sequence, each writes its output normalised by its own sum
// (fp16, plus its max and sum in float32) and a second kernel merges them;
// the workgroups of one sequence are placed on one XCD so the query reads
// and the partials stay in that XCD's L2.
#include "common.h"
#include "internal.h"
#include "select.h"
#include "stream_select.h"

namespace csa2 {
namespace {

constexpr int kTile = 32;                   // key slots per tile
// fp16 per Kt row: 1024 bytes + 32 bytes of padding.  With a 16-byte pad
// the logit operand reads (lane (c, q4) at row c, chunk q4 + 4s) take two
// LDS cycles per 16 lanes on gfx950 (measured: 1.66x the time of
// contiguous reads); with 32 bytes they take one.
constexpr int kKtStride = 528;
constexpr int kKtElems = kTile * kKtStride;
constexpr int kBufElems = kKtElems;         // one key-major tile per buffer
constexpr int kSmemBytes = 2 * kBufElems * 2 + 2 * kTile * 4;
// The epilogue stages 4 waves x 16 heads x (512 + 8) halfs in the same LDS.
static_assert(4 * 16 * (512 + 8) * 2 <= kSmemBytes, "output staging fits");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;       // log2 units

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f16x2_bits(f16x2_t v) {
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f16x2_t bits_f16x2(uint32_t v) {
  return __builtin_bit_cast(f16x2_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return bf2_bits(v);
}


// Rotation of RoPE pair i at query position t by -t * w (w = the pair's
// frequency, computed on the host in double): the angle is formed and
// reduced modulo 2 pi in double (t * w reaches about 1e6 rad at a million
// positions), then the cosine and sine of the remainder in float.
__device__ __forceinline__ void rope_cs(int32_t t, double w, float& c,
                                        float& s) {
  constexpr double kTwoPiHi = 6.283185307179586;          // 2 pi, head
  constexpr double kTwoPiLo = 2.4492935982947064e-16;     // 2 pi, tail
  const double ang = -(double)t * w;
  const double kq = rint(ang * (1.0 / kTwoPiHi));
  double r = fma(-kq, kTwoPiHi, ang);
  r = fma(-kq, kTwoPiLo, r);
  sincosf((float)r, &s, &c);
}

// (x, y) -> (x c - y s, x s + y c): the rotation of one pair.
__device__ __forceinline__ void rotate_pair(float& x, float& y, float c,
                                            float s) {
  const float nx = x * c - y * s;
  const float ny = x * s + y * c;
  x = nx;
  y = ny;
}

// Kernel arguments.  A workgroup's first accesses to this block miss the
// scalar cache one 64-byte line at a time, each a full memory latency, so
// what the start of the kernel needs (the workgroup mapping, the query, the
// window length and the fused selection's candidates) shares the first
// line, and the epilogue's rotation table comes last.
struct AttnArgs {
  int B;
  int splits;
  int k;
  int n_wg, kloc;          // fused selection: groups and pairs per group
  int tiles_per_split;
  const uint16_t* q;
  const int32_t* n_swa;
  const uint2* lcand;      // [B][n_wg][kloc] (key, id), id order
  const uint32_t* lbound;  // [B][n_wg]
  // -- 64 bytes
  const uint8_t* main_codes;
  const uint8_t* main_scales;
  int64_t n_cap;
  const int32_t* topk;
  const uint8_t* swa;
  float scale_log2;        // scale * log2(e)
  int n_tiles;
  int n_main;              // tiles holding chosen entries: ceil(k / 32)
  uint16_t* out;           // final output when splits == 1
  uint16_t* part_o;        // [B][S][64][512] fp16, normalised per split
  float* part_ml;          // [B][S][64][2] (max in log2 units, sum)
  // Fused selection (the decode path): every workgroup selects its
  // sequence's top-k itself from the indexer's local candidates.
  const uint32_t* keys;    // [B][ld] selection keys (exact fallback)
  int64_t ld;
  const int32_t* n_entries;
  const int32_t* fb_ids;   // [B][fb_n] entry ids of the key rows, or null
  int64_t fb_n;
  int n_div;               // entries per key row of the fallback (blocks)
  int32_t* topk_out;       // [B][k], written by each sequence's split 0
  AttnEpilogue epi;        // sink and de-rotation (final output only)
};
static_assert(offsetof(AttnArgs, lbound) + sizeof(void*) <= 64,
              "the kernel's first accesses share one line");

// The fields before the 64-byte mark are also passed ahead of the struct as
// plain arguments (14 dwords): the build preloads a kernel's leading
// scalar arguments into scalar registers at dispatch (a struct argument is
// not preloaded), so the kernel's first steps need no argument load.  The
// kernel puts them back into a local copy of the struct; that copy's `epi`
// is not used (it holds an array indexed per lane, which would put the
// copy in scratch memory): the epilogue reads the argument struct's own.
#define CSA2_ATTN_HEAD_PARAMS                                                \
  int h_B, int h_splits, int h_k, int h_n_wg, int h_kloc, int h_tps,         \
      const uint16_t *h_q, const int32_t *h_n_swa, const uint2 *h_lcand,     \
      const uint32_t *h_lbound
#define CSA2_ATTN_HEAD_ARGS(a)                                               \
  (a).B, (a).splits, (a).k, (a).n_wg, (a).kloc, (a).tiles_per_split, (a).q,  \
      (a).n_swa, (a).lcand, (a).lbound
#define CSA2_ATTN_HEAD_RESTORE(p, a)                                         \
  AttnArgs p = (a);                                                          \
  p.B = h_B;                                                                 \
  p.splits = h_splits;                                                       \
  p.k = h_k;                                                                 \
  p.n_wg = h_n_wg;                                                           \
  p.kloc = h_kloc;                                                           \
  p.tiles_per_split = h_tps;                                                 \
  p.q = h_q;                                                                 \
  p.n_swa = h_n_swa;                                                         \
  p.lcand = h_lcand;                                                         \
  p.lbound = h_lbound

// Shared memory of the fused selection (512 threads), overlaid on the
// attention's tile buffers, which are not in use yet: the candidate pass,
// and over it the exact fallback's streaming store.
template <int NC>
struct CandSmemT {
  int32_t hist[4][256];             // one histogram per narrowing pass
  uint32_t red[4][8];
  uint2 stage[NC];                  // the candidates, in their global order
};
template <int NC>
struct FselSmemT {
  union {
    CandSmemT<NC> cand;
    struct {
      uint32_t key[512 * kStreamPer];
      int32_t id[512 * kStreamPer];
      SelSmem<512, 256> sel;
    };
  };
};
using FselSmem = FselSmemT<4096>;     // the attention kernel's
constexpr int kMaxK = 2048;

// Raw gather registers for the 8 slots this lane dequantises in one tile.
// They hold the loaded words untouched, so nothing waits for the loads
// before the dequantisation that consumes them.
struct Raw {
  uint32_t a[8];
  uint32_t c[8];
};

// Slot (within a tile) of this lane's e-th element: wavefront `quarter`
// owns slots {4q..4q+3, 16+4q..16+4q+3}, lane g owns dims 8g..8g+7.
__device__ __forceinline__ int slot_of(int quarter, int e) {
  return e < 4 ? 4 * quarter + e : 16 + 4 * quarter + (e - 4);
}

// Top-k ids of this wavefront's slots, loaded by every lane with a
// per-lane (vector) load: a scalar load would share its wait counter with the
// LDS reads of the products and stall them.  Lane l fetches slot (l & 7) of
// tile `ta` (l < 8) or `tb` (l >= 8).  Slots past the chosen entries read a
// clamped, always valid address; their value is unused.  `ids` is the
// sequence's id row: in global memory, or in LDS after a fused selection.
__device__ __forceinline__ int32_t load_ids(const AttnArgs& p,
                                            const int32_t* ids, int ta,
                                            int tb, int quarter, int lane) {
  const int slot = ((lane & 8) ? tb : ta) * kTile + slot_of(quarter, lane & 7);
  return ids[slot < p.k ? slot : 0];
}

// Key rows of the fused selection's exact fallback: positions are the entry
// ids, or `idrow` names them (a pool's rows; ids ascending where valid, -1
// rows taking key 0).
struct FallbackSrc {
  const uint32_t* row;
  const int32_t* idrow;
  __device__ __forceinline__ void load(int64_t i, uint32_t& r,
                                       int32_t& id) const {
    r = row[i];
    id = idrow ? idrow[i] : (int32_t)i;
  }
  __device__ static __forceinline__ uint32_t key(uint32_t r) { return r; }
};

// The fused selection: the exact top-k of sequence b from the indexer's
// local candidates (the k largest pair keys, equal keys to the lower id,
// since the pairs are in id order), into sel_ids[0..k) ascending with -1
// padding, and into topk_out by split 0.  It is exact when the k-th largest
// candidate key is above every group's bound L (nothing a group left out can
// then reach the top k), or, with fewer than k valid candidates, when no
// group left anything out; otherwise the whole row's selection keys are
// streamed through the exact block selection instead.  So only candidates
// above L can matter: with at least k of them, their top k is the answer;
// with fewer, it is all of them when L = 0, else the fallback decides.
//
// The k-th key is found by narrowing [lo, hi] = [L + 1, max] with 256-bin
// histograms (a fresh one per pass, so none is cleared in between): each
// pass bins the keys still inside, and every wavefront scans the bins and
// narrows to the bin where the count from the top reaches the number still
// needed (the first pass also gives the count above L).  It ends on a bin
// holding exactly that number, or on one key value (ties then go to the
// lower positions).  One block scan places the chosen pairs in id order.
// All 512 threads take part; ends with a barrier.  Only LDS is written here:
// a global store before that barrier would make every wavefront wait at it
// for the store to complete, so the ids go to topk_out at the kernel's end.
// `after_stage` runs once the candidates are staged and every fetched value
// has arrived: loads it issues (the attention's query) are not waited for
// here, and they do not hold up the candidates (see the kernel).
struct NoLoads {
  __device__ __forceinline__ void operator()() const {}
};
template <int PER, typename Smem, typename After = NoLoads>
__device__ __forceinline__ void fused_select(const AttnArgs& p, int b,
                                             int32_t* sel_ids, Smem& fs,
                                             After after_stage = {}) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto& cs = fs.cand;
  static_assert(PER * 512 <= (int)(sizeof(cs.stage) / sizeof(uint2)),
                "the candidate stage holds every pair");
  if (tid < 256) reinterpret_cast<int4*>(&cs.hist[0][0])[tid] = make_int4(0, 0, 0, 0);
  const int C = p.n_wg * p.kloc;
  const uint2* cr = p.lcand + (int64_t)b * C;
  // The candidates arrive in coalesced passes (pass j: pairs 512j + tid)
  // and go through LDS, so that thread tid then holds pairs PER*tid ..
  // PER*tid+PER-1, consecutive in id order.  Read straight into that order,
  // every wavefront load would touch 32 cache lines for 512 bytes.
  uint2 v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = 512 * j + tid;
    v[j] = cr[i < C ? i : C - 1];
  }
  // One bound per thread (n_wg <= kLocalMaxCands / 8 = 512), loaded
  // unconditionally from a clamped index so nothing waits for it yet.
  static_assert(kLocalMaxCands / 8 <= 512, "one bound per thread");
  const uint32_t lbv =
      p.lbound[(int64_t)b * p.n_wg + (tid < p.n_wg ? tid : p.n_wg - 1)];
  uint32_t lb = tid < p.n_wg ? lbv : 0u, km = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (512 * j + tid < C) km = max(km, v[j].x);
    cs.stage[512 * j + tid] = v[j];
  }
  // Every fetched value is in (the bound is used here), so the loads issued
  // next are never waited for before the first barrier.
  asm volatile("" : : "v"(lb));
  after_stage();
  lb = wave_max_u32(lb);
  km = wave_max_u32(km);
  if (lane == 0) {
    cs.red[0][wv] = lb;
    cs.red[1][wv] = km;
  }
  __syncthreads();
  uint32_t kk[PER];
  int32_t ci[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    const uint2 w = cs.stage[i];
    kk[j] = i < C ? w.x : 0u;
    ci[j] = (int32_t)w.y;
  }
  uint32_t L = 0u, MX = 0u;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    L = max(L, cs.red[0][w]);
    MX = max(MX, cs.red[1][w]);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) kk[j] = kk[j] > L ? kk[j] : 0u;
  const int k = p.k;
  uint32_t lo = L + 1u, hi = MX;
  int need = k, n = 0;
  bool take_all = MX <= L;            // no key above L
  for (int it = 0; it < 4 && !take_all && lo < hi; ++it) {
    int32_t* H = cs.hist[it];
    const int bits = 32 - __builtin_clz(hi - lo);
    const int shift = bits > 8 ? bits - 8 : 0;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if ((kk[j] >= lo) & (kk[j] <= hi)) atomicAdd(&H[(hi - kk[j]) >> shift], 1);
    __syncthreads();
    // Lane L holds bins 4L .. 4L+3 (bins in key order from the top).
    const int4 c = reinterpret_cast<const int4*>(H)[lane];
    const int sc = c.x + c.y + c.z + c.w;
    const int incl = wave_incl_scan(sc);
    if (it == 0) {
      n = __builtin_amdgcn_readlane(incl, 63);
      if (n <= k) { take_all = true; break; }
    }
    const int run = incl - sc;
    const bool hit = (run < need) & (run + sc >= need);
    const int hl = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(hit));
    int bi = 0, before = run, cnt = c.x;
    if (before + c.x < need) {
      before += c.x; bi = 1; cnt = c.y;
      if (before + c.y < need) {
        before += c.y; bi = 2; cnt = c.z;
        if (before + c.z < need) { before += c.z; bi = 3; cnt = c.w; }
      }
    }
    const int bs = __builtin_amdgcn_readlane(4 * lane + bi, hl);
    need -= __builtin_amdgcn_readlane(before, hl);
    const bool exact = __builtin_amdgcn_readlane(cnt, hl) == need;
    const uint32_t nhi = hi - ((uint32_t)bs << shift);
    const uint32_t width = (1u << shift) - 1u;
    lo = nhi - lo >= width ? nhi - width : lo;
    hi = nhi;
    if (exact) { take_all = true; break; }
  }
  if (MX > L && lo == hi && !take_all && n == 0) {
    // One key value above L (the loop never ran): it is the k-th key when
    // at least k keys hold it.
    n = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) n += kk[j] != 0u;
    n = __builtin_amdgcn_readlane(wave_incl_scan(n), 63);
    if (lane == 0) cs.red[2][wv] = (uint32_t)n;
    __syncthreads();
    n = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) n += (int)cs.red[2][w];
    take_all = n <= k;
  }
  const bool ok = take_all ? (n >= k || L == 0u) : true;
  if (ok) {
    // Chosen: take_all -> every key >= lo (all keys above L when the first
    // pass took them all); else keys > hi (= lo) plus the first `need` keys
    // equal to lo.  One packed scan (ties << 16 | greater).
    // (lo >= L + 1 >= 1 here, so a zeroed key is never chosen; the loops
    // below are branch-free: a key's place, or a spare slot past k.)
    int ngt = 0, ntie = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t key = kk[j];
      ngt += (key != 0u) & (take_all ? key >= lo : key > hi);
      ntie += (key != 0u) & !take_all & (key == lo);
    }
    const int x = (ntie << 16) | ngt;
    const int incl = wave_incl_scan(x);
    if (lane == 63) cs.red[3][wv] = (uint32_t)incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int t = (int)cs.red[3][w];
      before += w < wv ? t : 0;
      tot += t;
    }
    const int ex = before + incl - x;
    const int gt_before = ex & 0xFFFF, tie_before = ex >> 16;
    int tie_rank = tie_before;
    int q = gt_before + (take_all ? 0 : min(tie_before, need));
    const int total = (tot & 0xFFFF) + (take_all ? 0 : min(tot >> 16, need));
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t key = kk[j];
      const bool gt = (key != 0u) & (take_all ? key >= lo : key > hi);
      const bool tie = (key != 0u) & !take_all & (key == lo);
      const bool sel = gt | (tie & (tie_rank < need));
      tie_rank += tie;
      sel_ids[sel ? q : kMaxK] = ci[j];
      q += sel;
    }
    for (q = total + tid; q < k; q += 512) sel_ids[q] = -1;
  } else {
    // The exact streaming selection over the whole key row (its store
    // overlays the candidate state, so start behind a barrier).
    __syncthreads();
    for (int i = tid; i < 8 * 256; i += 512) (&fs.sel.hist[0][0])[i] = 0;
    __syncthreads();
    int64_t len = p.fb_n;
    if (p.fb_ids == nullptr) {
      // Visible rows: n_entries[b], or ceil(n_entries[b] / n_div) blocks.
      const int32_t ne = p.n_entries[b];
      len = ne <= 0 ? 0 : ((int64_t)ne + p.n_div - 1) / p.n_div;
      len = len < p.n_cap ? len : p.n_cap;
    }
    const FallbackSrc src{p.keys + (int64_t)b * p.ld,
                          p.fb_ids ? p.fb_ids + (int64_t)b * p.fb_n : nullptr};
    const int cnt = stream_select<512>(fs, len, p.k, src);
    for (int q = tid; q < p.k; q += 512) sel_ids[q] = q < cnt ? fs.id[q] : -1;
  }
  __syncthreads();
}

// Per-sequence bases of the gathered planes (wavefront-uniform).
struct Bases {
  const uint8_t* codes;    // main codes of the sequence
  const uint8_t* scales;   // main scales of the sequence
  const uint8_t* swa;      // window rows of the sequence
};

// Issue the two dword loads of each of this wavefront's 8 slots of `tile`:
// main entry -> code dword + the dword holding its scale byte, window row ->
// its 8 bytes; `kinds` records per slot 0 = empty, 1 = main entry, 2 =
// window row (empty slots read row 0).  Lane off+e (e < 8) holds slot e's
// id in `idl` and works out that slot's byte offsets and kind with vector
// arithmetic; each load then takes a uniform base plus a 32-bit lane offset
// (row offsets within one sequence stay below 2^32 since n_cap <= 2^24).
__device__ __forceinline__ void load_rows(const AttnArgs& p, const Bases& bs,
                                          int tile, int quarter, int lane,
                                          int nswa, int32_t idl, int off,
                                          Raw& raw, uint32_t& kinds) {
  const int g = lane;
  const int slot_l = tile * kTile + slot_of(quarter, lane & 7);
  const bool main_l = slot_l < p.k;
  const bool ok_main = main_l && (uint32_t)idl < (uint32_t)p.n_cap;
  const int rr = slot_l - p.k;
  const bool ok_swa = !main_l && rr < nswa;
  const uint32_t row = ok_main ? (uint32_t)idl : 0u;
  const uint32_t srow = ok_swa ? (uint32_t)rr : 0u;
  const uint32_t offa = main_l ? row * 256u : srow * 512u;
  const uint32_t offc = main_l ? row * 32u : srow * 512u + 4u;
  const uint32_t g4 = 4u * (uint32_t)g, g8 = 8u * (uint32_t)g;
  const uint32_t gs = (uint32_t)((g >> 1) & ~3);
  // Slot kinds from two ballots (bit e: slot e, held by lane off+e), each
  // bit spread to the low bit of a 2-bit field: 1 = chosen entry, 2 =
  // window row (exclusive), 0 = empty.
  auto spread = [](uint32_t x) {
    x = (x | (x << 4)) & 0x0F0Fu;
    x = (x | (x << 2)) & 0x3333u;
    return (x | (x << 1)) & 0x5555u;
  };
  const uint32_t mm =
      (uint32_t)(__builtin_amdgcn_ballot_w64(ok_main) >> off) & 0xFFu;
  const uint32_t ms =
      (uint32_t)(__builtin_amdgcn_ballot_w64(ok_swa) >> off) & 0xFFu;
  kinds = spread(mm) | (spread(ms) << 1);
  if (tile * kTile + 16 + 4 * quarter + 3 < p.k) {
    // All 8 slots of this wavefront are chosen entries (every tile before
    // the one holding slot k): no per-slot choice of plane or offset.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t oa = __builtin_amdgcn_readlane(offa, off + e);
      const uint32_t oc = __builtin_amdgcn_readlane(offc, off + e);
      raw.a[e] = *reinterpret_cast<const uint32_t*>(bs.codes + (oa + g4));
      raw.c[e] = *reinterpret_cast<const uint32_t*>(bs.scales + (oc + gs));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool is_main = tile * kTile + slot_of(quarter, e) < p.k;
      const uint32_t oa = __builtin_amdgcn_readlane(offa, off + e);
      const uint32_t oc = __builtin_amdgcn_readlane(offc, off + e);
      const uint8_t* ba = is_main ? bs.codes : bs.swa;
      const uint8_t* bc = is_main ? bs.scales : bs.swa;
      raw.a[e] = *reinterpret_cast<const uint32_t*>(ba + (oa + (is_main ? g4 : g8)));
      raw.c[e] = *reinterpret_cast<const uint32_t*>(bc + (oc + (is_main ? gs : g8)));
    }
  }
}

// Dequantise the gathered slots (exactly, to fp16) and write both LDS
// layouts of one buffer.
__device__ __forceinline__ void dequant_store(const Raw& raw, uint32_t kinds,
                                              int quarter, int g,
                                              _Float16* buf, int32_t* valid) {
  uint32_t kd[8][4];
  // The slot kinds are the same in every lane.  A wavefront whose 8 slots
  // are all chosen entries or all window rows (every tile but the one
  // holding slot k, when the ids are valid and the window is full) takes
  // one straight-line path; others decide per slot.
  auto main_slot = [&](int e) {
    // (s, s) in fp16 from the E4M3 scale byte duplicated into two lanes.
    const uint32_t sb = (raw.c[e] >> (8 * ((g >> 1) & 3))) & 0xFFu;
    const f16x2_t ss = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
        sb * 0x101u, 1.0f, false);
    const uint32_t cw = raw.a[e];
    kd[e][0] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * ss);
    kd[e][1] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * ss);
    kd[e][2] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * ss);
    kd[e][3] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * ss);
  };
  auto window_slot = [&](int e) {
    kd[e][0] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.a[e], 1.0f, false));
    kd[e][1] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.a[e], 1.0f, true));
    kd[e][2] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.c[e], 1.0f, false));
    kd[e][3] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.c[e], 1.0f, true));
  };
  if (kinds == 0x5555u) {
#pragma unroll
    for (int e = 0; e < 8; ++e) main_slot(e);
  } else if (kinds == 0xAAAAu) {
#pragma unroll
    for (int e = 0; e < 8; ++e) window_slot(e);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t kind = (kinds >> (2 * e)) & 3u;
      if (kind == 1) {
        main_slot(e);
      } else if (kind == 2) {
        window_slot(e);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) kd[e][i] = 0;
      }
    }
  }
  // Key-major rows: slot j, dims 8g .. 8g+7.
  _Float16* kt = buf;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = slot_of(quarter, e);
    u32x4 v = {kd[e][0], kd[e][1], kd[e][2], kd[e][3]};
    *reinterpret_cast<u32x4*>(kt + j * kKtStride + 8 * g) = v;
  }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = slot_of(quarter, e);
      valid[j] = ((kinds >> (2 * e)) & 3u) != 0;
    }
  }
}

// Workgroup -> (sequence, split), placing all splits of a sequence on one
// XCD: workgroups are dealt to the 8 XCDs round-robin by their linear id
// (from a starting XCD that rotates between launches), so the ids of one
// sequence, which agree mod 8, land on one XCD.
__device__ __forceinline__ bool map_workgroup(int id, int B, int S, int& b,
                                              int& split) {
  const int xcd = id & 7, slot = id >> 3;
  b = xcd + 8 * (slot / S);
  split = slot % S;
  return b < B;
}

// A split's tiles in the order it runs them.  With given ids (no fused
// selection) the pure window tiles (n_main .. n_tiles-1, rows that need no
// ids) are dealt first, one to each of the first splits, and the chosen
// entries' tiles evenly after them (any remainder to the last splits): a
// split that starts on window rows gathers them while its first ids load,
// which takes one memory round trip out of its prologue.  After a fused
// selection the ids are in LDS and the splits take contiguous ranges of
// tiles_per_split tiles.
struct TileMap {
  int w_cnt, wbase, S, m0, cnt;
  __device__ __forceinline__ int phys(int t) const {
    return t < w_cnt ? wbase + S * t : m0 + (t - w_cnt);
  }
};
template <bool FSEL>
__device__ __forceinline__ TileMap tile_map(const AttnArgs& p, int split) {
  TileMap m;
  const int S = p.splits;
  m.S = S;
  if constexpr (FSEL) {
    m.w_cnt = 0;
    m.wbase = 0;
    m.m0 = split * p.tiles_per_split;
    const int end = m.m0 + p.tiles_per_split;
    m.cnt = (end < p.n_tiles ? end : p.n_tiles) - m.m0;
    if (m.cnt < 0) m.cnt = 0;
  } else {
    const int n_win = p.n_tiles - p.n_main;
    m.w_cnt = split < n_win ? (n_win - split + S - 1) / S : 0;
    m.wbase = p.n_main + split;
    const int base = p.n_main / S, extra = p.n_main % S;
    const int first_extra = S - extra;
    m.m0 = split * base + (split > first_extra ? split - first_extra : 0);
    m.cnt = m.w_cnt + base + (split >= first_extra ? 1 : 0);
  }
  return m;
}

struct TileState {
  f32x4 acc[32];           // O^T accumulators: dims 16*blk + 4*q4 + r
  float m_run;             // exp2 reference point (log2 units)
  float l_run;             // running sum of this lane's weights
  float scale;             // logit scale of this lane's head (log2 units,
                           // times the head's query prescale)
};

// Producer side of one key tile (wavefronts 4..7, `quarter` = wavefront - 4).
// P = parity of the tile within the split: raw[P] is free again (its rows
// went to LDS in the previous step) and receives the rows of tile t+2, with
// the ids of t+3 issued first (wait counts retire in order, so reading them
// next step does not wait for these rows); then raw[P^1] (rows of t+1) is
// dequantised into LDS buffer P^1 while the math wavefronts read buffer P.
template <int P>
__device__ __forceinline__ void tile_produce(
    const AttnArgs& p, const Bases& bs, const int32_t* ids, const TileMap& tm,
    int t, int t1, int quarter, int lane, int nswa, _Float16* bufs,
    int32_t* valid_base, Raw (&raw)[2], uint32_t (&kinds)[2], int32_t& idn) {
  const int tl = t1 - 1;
  const int t3 = tm.phys(t + 3 < t1 ? t + 3 : tl);
  const int32_t id3 = load_ids(p, ids, t3, t3, quarter, lane);
  load_rows(p, bs, tm.phys(t + 2 < t1 ? t + 2 : tl), quarter, lane, nswa, idn,
            0, raw[P], kinds[P]);
  idn = id3;
  if (t + 1 < t1)
    dequant_store(raw[P ^ 1], kinds[P ^ 1], quarter, lane,
                  bufs + (P ^ 1) * kBufElems, valid_base + (P ^ 1) * kTile);
}

// Math side of one key tile (wavefronts 0..3): logits, online softmax and
// the value products over LDS buffer P.
template <int P>
__device__ __forceinline__ void tile_math(
    const AttnArgs& p, int col, int q4, const _Float16* bufs,
    const int32_t* valid_base, const f16x8_t (&qb)[16], TileState& st) {
  const _Float16* kt = bufs + P * kBufElems;
  const int32_t* valid = valid_base + P * kTile;

  // S^T = K Q^T for the 32 slots of this tile, as four independent
  // accumulation chains (slot halves x even/odd k-steps).  Operands are read
  // kAhead steps before their products, so LDS latency overlaps the
  // matrix-core work (the scheduling barriers keep that order).
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  {
    f32x4 s0b = {0.f, 0.f, 0.f, 0.f}, s1b = {0.f, 0.f, 0.f, 0.f};
    constexpr int kAhead = 2;
    const _Float16* k0 = kt + col * kKtStride + 8 * q4;
    const _Float16* k1 = k0 + 16 * kKtStride;
    f16x8_t a0[kAhead], a1[kAhead];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) {
      a0[s] = *reinterpret_cast<const f16x8_t*>(k0 + 32 * s);
      a1[s] = *reinterpret_cast<const f16x8_t*>(k1 + 32 * s);
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const f16x8_t c0 = a0[s % kAhead], c1 = a1[s % kAhead];
      if (s + kAhead < 16) {
        a0[s % kAhead] = *reinterpret_cast<const f16x8_t*>(k0 + 32 * (s + kAhead));
        a1[s % kAhead] = *reinterpret_cast<const f16x8_t*>(k1 + 32 * (s + kAhead));
      }
      if (s & 1) {
        s0b = __builtin_amdgcn_mfma_f32_16x16x32_f16(c0, qb[s], s0b, 0, 0, 0);
        s1b = __builtin_amdgcn_mfma_f32_16x16x32_f16(c1, qb[s], s1b, 0, 0, 0);
      } else {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(c0, qb[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(c1, qb[s], s1, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s0 += s0b;
    s1 += s1b;
  }
  // Logits in log2 units; lane holds slots 4*q4 + r and 16 + 4*q4 + r.
  float x[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = valid[4 * q4 + r] ? s0[r] * st.scale : -__builtin_inff();
    x[4 + r] = valid[16 + 4 * q4 + r] ? s1[r] * st.scale : -__builtin_inff();
  }
  float mt = x[0];
#pragma unroll
  for (int r = 1; r < 8; ++r) mt = fmaxf(mt, x[r]);
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  // Move the reference point when the tile maximum rises by more than the
  // slack (also from -inf).  Nothing has been accumulated while it is still
  // -inf, so only a head with history rescales its accumulators.
  const bool bump = mt > st.m_run + kRescaleSlack;
  const bool rescale = bump & (st.m_run != -__builtin_inff());
  if (__any(rescale)) {
    if (rescale) {
      const float alpha = exp2f(st.m_run - mt);
      st.l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) st.acc[i] *= alpha;
    }
  }
  if (bump) st.m_run = mt;
  const float mref = st.m_run == -__builtin_inff() ? 0.0f : st.m_run;
  f16x8_t pb;
#pragma unroll
  for (int r = 0; r < 8; ++r) pb[r] = (_Float16)exp2f(x[r] - mref);
  // The running sum takes the same rounded weights the product uses.
#pragma unroll
  for (int r = 0; r < 8; ++r) st.l_run += (float)pb[r];

  // O^T += V^T P^T, V^T read from the key-major tile by transposing LDS
  // reads (ds_read_b64_tr_b16): within a 16-lane group, lane i receives
  // element i mod 4 of the 8-byte chunks addressed by lanes 4j + i/4
  // (j = 0..3).  The product's k index for lane group q4 runs over slots
  // 4*q4 .. 4*q4+3 and then 16+4*q4 .. 16+4*q4+3 (the logits' output
  // order, which is how the probabilities arrive), so lane m of group q4
  // addresses row 4*q4 + m/4 (then 16 rows further) at dims
  // 16*blk + 4*(m mod 4): lane i = col receives dim 16*blk + col of those
  // eight slots.  Two bases per lane, a 32-byte immediate step per block.
  {
    constexpr int kAhead = 4;
    const _Float16* ta0 =
        kt + (4 * q4 + (col >> 2)) * kKtStride + 4 * (col & 3);
    const _Float16* ta1 = ta0 + 16 * kKtStride;
    auto v_operand = [&](int blk) -> f16x8_t {
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(ta0 + 16 * blk));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(ta1 + 16 * blk));
      return __builtin_bit_cast(
          f16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    f16x8_t va[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) va[i] = v_operand(i);
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) {
      const f16x8_t c = va[blk % kAhead];
      if (blk + kAhead < 32) va[blk % kAhead] = v_operand(blk + kAhead);
      st.acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(c, pb, st.acc[blk], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

}

// Dynamic shared memory: the tile buffers (overlaid by the fused
// selection's store first), then the selected ids of a fused selection.
constexpr int kFselBytes = (int)sizeof(FselSmem);
constexpr int kUnionBytes = (kSmemBytes > kFselBytes ? kSmemBytes : kFselBytes);
constexpr int kFusedSmemBytes = kUnionBytes + (kMaxK + 64) * 4;  // + spare

template <bool FSEL, int CPER>
__global__ __launch_bounds__(512, 1) void attn_kernel(CSA2_ATTN_HEAD_PARAMS,
                                                      AttnArgs args) {
  CSA2_ATTN_HEAD_RESTORE(p, args);
  extern __shared__ __align__(16) uint8_t smem_raw[];
  _Float16* bufs = reinterpret_cast<_Float16*>(smem_raw);
  int32_t* valid_base = reinterpret_cast<int32_t*>(smem_raw + 2 * kBufElems * 2);

  int b, split;
  if (!map_workgroup(blockIdx.x, p.B, p.splits, b, split)) return;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Wavefronts 0..3 are the math side (wavefront w: heads 16w..16w+15, its
  // queries and accumulators in registers); 4..7 the producers (gather and
  // dequantisation, producer q handling slot quarter q of every tile).  Each
  // SIMD holds one of each, so the matrix work of one tile overlaps the
  // gather and dequantisation of the next.
  const bool is_math = wv < 4;
  const int wave = wv & 3;
  const int col = lane & 15;          // head within the wave / row in A
  const int q4 = lane >> 4;           // k-slot group
  const int head = 16 * wave + col;
  // The window length is loaded per lane (the zero offset is hidden from
  // the compiler, which would otherwise use a scalar load and wait for it
  // at once to free its register): its latency then overlaps the
  // selection instead of delaying the candidate loads.
  int zero = 0;
  asm volatile("" : "+v"(zero));
  const int nswa_raw = p.n_swa[b + zero];
  const int nswa = nswa_raw < 0 ? 0 : (nswa_raw > kWindow ? kWindow : nswa_raw);

  const TileMap tm = tile_map<FSEL>(p, split);
  const int t0 = 0, t1 = tm.cnt;
  const bool wfirst = tm.w_cnt > 0;   // the first tile is window rows

  // Gather pipeline (producers): while tile t runs on the matrix cores, the
  // rows of tiles t+1 and t+2 are in flight (a two-slot register ring, slot
  // = parity of the tile within the split) and the ids of tile t+3 behind
  // them.  Tile indices past the split are clamped to its last tile, so
  // every load is unconditional and valid.
  const Bases bs{p.main_codes + (int64_t)b * p.n_cap * 256,
                 p.main_scales + (int64_t)b * p.n_cap * 32,
                 p.swa + (int64_t)b * kWindow * 512};
  const int tl = t1 - 1;
  const int ta = t0 < t1 ? t0 : tl < 0 ? 0 : tl;
  const int tb = t0 + 1 < t1 ? t0 + 1 : ta;
  Raw raw[2];
  uint32_t kinds[2] = {0u, 0u};
  int32_t idn = 0;
  TileState st;
  f16x8_t qb[16];
  // The sequence's id row: global (given top-k) or, after a fused
  // selection, LDS.
  int32_t* sel_ids = reinterpret_cast<int32_t*>(smem_raw + kUnionBytes);
  const int32_t* ids = FSEL ? sel_ids : p.topk + (int64_t)b * p.k;
  // Q^T operand: head `head`, dims 32s + 8*q4 .. +7.  With a fused
  // selection the raw query is issued only once the candidates are in, and
  // arrives during the selection.  Issued first, its 64 KB per workgroup
  // queued ahead of the candidate loads in the CU's memory pipeline: a
  // phase probe (encoder-full-64k) put the candidate staging at ~6.5K
  // cycles after the start, against ~4.1K this way (step -1.6 us).
  bf16x8_t qraw[16];
  auto load_query = [&]() {
    if (is_math) {
      const bf16x8_t* qr = reinterpret_cast<const bf16x8_t*>(
          p.q + ((int64_t)b * kHeads + head) * 512 + 8 * q4);
#pragma unroll
      for (int s = 0; s < 16; ++s) qraw[s] = qr[4 * s];
    }
  };
  if constexpr (FSEL)
    fused_select<CPER>(p, b, sel_ids, *reinterpret_cast<FselSmem*>(smem_raw),
                       load_query);
  else
    load_query();
  if (is_math) {
    // The query converted to fp16 after a power-of-two prescale per head
    // (exact): the head's largest |q| lands in [2^14, 2^15), so no bf16
    // value overflows fp16 and values within 2^28 of the largest convert
    // exactly; the logit scale takes the inverse factor.  The prescale
    // exponent is clamped to [-100, 64] (heads with max |q| >= 2^79 are
    // outside the supported range).  The accumulators are zeroed after the
    // conversion (the raw query is dead by then).
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)qraw[s][j]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int ex = 0;
    if (amax > 0.0f) frexpf(amax, &ex);          // amax < 2^ex
    const int e = amax > 0.0f ? min(max(ex - 15, -100), 64) : 0;
    const float qs = ldexpf(1.0f, -e);
    st.scale = p.scale_log2 * ldexpf(1.0f, e);
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) qb[s][j] = (_Float16)((float)qraw[s][j] * qs);
#pragma unroll
    for (int s = 0; s < 16; ++s) asm volatile("" : : "v"(qb[s]));
#pragma unroll
    for (int i = 0; i < 32; ++i) st.acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_run = -__builtin_inff();
    st.l_run = 0.0f;
  } else {
    // The rows of the first two tiles go out together (a producer holds no
    // accumulators, so nothing else wants their registers); the first is
    // dequantised into buffer 0.
    // A first tile of window rows needs no ids: its rows go out first.
    if (wfirst)
      load_rows(p, bs, tm.phys(ta), wave, lane, nswa, 0, 0, raw[0], kinds[0]);
    const int32_t id01 = load_ids(p, ids, tm.phys(ta), tm.phys(tb), wave, lane);
    idn = load_ids(p, ids, tm.phys(t0 + 2 < t1 ? t0 + 2 : ta), 0, wave, lane);
    if (!wfirst)
      load_rows(p, bs, tm.phys(ta), wave, lane, nswa, id01, 0, raw[0],
                kinds[0]);
    load_rows(p, bs, tm.phys(tb), wave, lane, nswa, id01, 8, raw[1], kinds[1]);
    if (t0 < t1) dequant_store(raw[0], kinds[0], wave, lane, bufs, valid_base);
  }
  __syncthreads();

  // Each side runs its own loop (the producers' in-flight rows are not
  // live in the math loop); both pass the same number of barriers, one per
  // tile.  The role is uniform within a wavefront (wv comes from
  // readfirstlane), and the hardware barrier (s_barrier) releases once every
  // wavefront of the workgroup has arrived at a barrier, whichever barrier
  // instruction each executes, so the two loops stay in step.
  if (is_math) {
    for (int t = t0; t < t1; t += 2) {
      tile_math<0>(p, col, q4, bufs, valid_base, qb, st);
      __syncthreads();
      if (t + 1 < t1) {
        tile_math<1>(p, col, q4, bufs, valid_base, qb, st);
        __syncthreads();
      }
    }
  } else {
    for (int t = t0; t < t1; t += 2) {
      tile_produce<0>(p, bs, ids, tm, t, t1, wave, lane, nswa, bufs,
                      valid_base, raw, kinds, idn);
      __syncthreads();
      if (t + 1 < t1) {
        tile_produce<1>(p, bs, ids, tm, t + 1, t1, wave, lane, nswa, bufs,
                        valid_base, raw, kinds, idn);
        __syncthreads();
      }
    }
  }
  const bool final_out = p.splits == 1;
  // The output (final bf16, or this split's fp16 partial normalised by its
  // own sum -- a convex combination of keys, so |value| <= 2688 fits fp16
  // with 11 significant bits) is staged through LDS (free after the last
  // tile's barrier) so that every store writes 16 contiguous bytes per lane
  // and whole 1 KB head rows per instruction.
  constexpr int kRowH = 512 + 8;                 // staged row, +16 B pad
  uint16_t* stg_all = reinterpret_cast<uint16_t*>(smem_raw);
  float m_run = 0.0f, l_tot = 0.0f;
  if (is_math) {
    f32x4 (&acc)[32] = st.acc;
    m_run = st.m_run;
    // Fold the running sums of the four lanes that share a head.
    l_tot = st.l_run + __shfl_xor(st.l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    // A sink logit joins the denominator of the final output (a split's
    // partial keeps its own sum; the merge adds the sink once).  With no key
    // at all (m_run = -inf) the output is zero either way.
    float den = l_tot;
    if (final_out && args.epi.sink != nullptr)
      den += exp2f(args.epi.sink[head] * kLog2e - m_run);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    if (final_out && args.epi.pos != nullptr) {
      // De-rotate dims 448..511 (blocks 28..31): this lane holds dims
      // 16*blk + 4*q4 + r, pairs (r = 0, 1) and (r = 2, 3).
      const int32_t t = args.epi.pos[b];
#pragma unroll
      for (int blk = 28; blk < 32; ++blk)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          float c, sn;
          rope_cs(t, args.epi.rope_w[8 * (blk - 28) + 2 * q4 + r / 2], c, sn);
          float x = acc[blk][r], y = acc[blk][r + 1];
          rotate_pair(x, y, c, sn);
          acc[blk][r] = x;
          acc[blk][r + 1] = y;
        }
    }
    // Head row h of the workgroup is staged at row h (the uniform choice of
    // format is made once, outside the unrolled loops, so each is
    // straight-line code).
    uint2* srow = reinterpret_cast<uint2*>(stg_all + head * kRowH + 4 * q4);
    if (final_out) {
#pragma unroll
      for (int blk = 0; blk < 32; ++blk)
        srow[4 * blk] = make_uint2(pack_bf16(acc[blk][0] * inv, acc[blk][1] * inv),
                                   pack_bf16(acc[blk][2] * inv, acc[blk][3] * inv));
    } else {
#pragma unroll
      for (int blk = 0; blk < 32; ++blk)
        srow[4 * blk] = make_uint2(
            f16x2_bits(f16x2_t{(_Float16)(acc[blk][0] * inv), (_Float16)(acc[blk][1] * inv)}),
            f16x2_bits(f16x2_t{(_Float16)(acc[blk][2] * inv), (_Float16)(acc[blk][3] * inv)}));
    }
  }
  __syncthreads();
  // All eight wavefronts store: wavefront w writes head rows 8w .. 8w+7.
  // The stores are nontemporal: the partials (14.7 MB over a 64K step) are
  // read back only by the next kernel, after this one has ended, and as
  // streaming writes they leave less in L2 to write back at the kernel's
  // end (step 41.3 -> 40.4 us).
  const int64_t row0 = final_out ? (int64_t)b * kHeads
                                 : ((int64_t)b * p.splits + split) * kHeads;
  uint16_t* dst = (final_out ? p.out : p.part_o) + row0 * 512 + 8 * lane;
#pragma unroll
  for (int h = 8 * wv; h < 8 * wv + 8; ++h)
    __builtin_nontemporal_store(
        *reinterpret_cast<const u32x4*>(stg_all + h * kRowH + 8 * lane),
        reinterpret_cast<u32x4*>(dst + h * 512));
  if (is_math && !final_out && q4 == 0) {
    const int64_t ps = ((int64_t)b * p.splits + split) * kHeads + head;
    p.part_ml[ps * 2 + 0] = m_run;
    p.part_ml[ps * 2 + 1] = l_tot;
  }
  // The selected ids (still in LDS: the staging above stays below them).
  if (FSEL && split == 0 && p.topk_out != nullptr)
    for (int q = threadIdx.x; q < p.k; q += 512)
      p.topk_out[(int64_t)b * p.k + q] = sel_ids[q];
}

// Merge of split partials: one wavefront per (sequence, head), lane d8
// merging dims 8*d8 .. 8*d8+7.  o = sum_s w_s o_s / sum_s w_s with
// w_s = l_s 2^(m_s - M).  The split count S is a template parameter, so the
// loads are straight-line code, all issued before any is used; the splits'
// maxima and sums are wavefront-uniform and come through scalar loads.
constexpr int kMaxSplits = 16;

template <int S>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml,
    int B, uint16_t* __restrict__ out, AttnEpilogue epi) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bh = (int64_t)blockIdx.x * 4 + wave;
  if (bh >= (int64_t)B * kHeads) return;       // wavefront-uniform
  const int d8 = threadIdx.x & 63;
  const int head = (int)(bh % kHeads);
  const int64_t b = bh / kHeads;
  float2 ml[S];
  u32x4 v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t ps = (b * S + s) * kHeads + head;
    ml[s] = *reinterpret_cast<const float2*>(part_ml + ps * 2);
    v[s] = *reinterpret_cast<const u32x4*>(part_o + ps * 512 + 8 * d8);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s].x);
  // A sink logit (log2 units here) joins the denominator once; the
  // reference point covers it too.
  const float z = epi.sink != nullptr ? epi.sink[head] * kLog2e
                                      : -__builtin_inff();
  M = fmaxf(M, z);
  const float mref = M == -__builtin_inff() ? 0.0f : M;
  float L = z == -__builtin_inff() ? 0.0f : exp2f(z - mref);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float wgt = ml[s].x == -__builtin_inff()
                          ? 0.0f : ml[s].y * exp2f(ml[s].x - mref);
    L += wgt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2_t h = bits_f16x2(v[s][i]);
      o[2 * i] += wgt * (float)h[0];
      o[2 * i + 1] += wgt * (float)h[1];
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if (epi.pos != nullptr && d8 >= 56) {
    // Dims 8*d8 .. 8*d8+7 are RoPE pairs 4*(d8-56) .. +3.
    const int32_t t = epi.pos[b];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float c, sn;
      rope_cs(t, epi.rope_w[4 * (d8 - 56) + j], c, sn);
      rotate_pair(o[2 * j], o[2 * j + 1], c, sn);
    }
  }
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16(o[2 * i] * inv, o[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(out + bh * 512 + 8 * d8) = w;
}

template <int S>
hipError_t launch_combine(const uint16_t* part_o, const float* part_ml,
                          int splits, int B, uint16_t* out,
                          const AttnEpilogue& epi, hipStream_t s) {
  if constexpr (S <= kMaxSplits) {
    if (splits != S)
      return launch_combine<S + 1>(part_o, part_ml, splits, B, out, epi, s);
    const int64_t waves = (int64_t)B * kHeads;
    hipLaunchKernelGGL(attn_combine_kernel<S>,
                       dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                       part_o, part_ml, B, out, epi);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;              // more splits than planned
  }
}

// Exact top-k of local candidates for a selection that no attention kernel
// follows: the blocks of the hierarchical pool.  One workgroup of 512
// threads per sequence runs the fused selection (its exact fallback streams
// the sequence's whole key row) and writes each chosen id expanded by
// `block` -- positions id*block .. id*block+block-1, those at or past
// limit[b] as -1 -- ascending, -1 padded to k*block.
using CandTopkSmem = FselSmemT<kCandTopkMax>;
constexpr int kCandTopkSmemBytes = (int)sizeof(CandTopkSmem) + (kMaxK + 64) * 4;

template <int CPER>
__global__ __launch_bounds__(512) void cand_topk_kernel(CSA2_ATTN_HEAD_PARAMS,
                                                        AttnArgs args,
                                                        int block,
                                                        const int32_t* limit,
                                                        int32_t* out) {
  CSA2_ATTN_HEAD_RESTORE(p, args);
  extern __shared__ __align__(16) uint8_t smem_raw[];
  int32_t* sel = reinterpret_cast<int32_t*>(smem_raw + sizeof(CandTopkSmem));
  const int b = blockIdx.x;
  fused_select<CPER>(p, b, sel, *reinterpret_cast<CandTopkSmem*>(smem_raw));
  // One chosen id per thread at a time: its `block` positions are
  // consecutive, so a block of 8 is two 16-byte stores (the rows of 32
  // threads in a row make one contiguous run).
  const int64_t lim = limit ? (int64_t)limit[b] : INT64_MAX;
  int32_t* o = out + (int64_t)b * p.k * block;
  for (int q = threadIdx.x; q < p.k; q += 512) {
    const int32_t id = sel[q];
    const int64_t base = (int64_t)id * block;
    auto at = [&](int t) -> int32_t {
      return (id >= 0 && base + t < lim) ? (int32_t)(base + t) : -1;
    };
    int32_t* dst = o + (int64_t)q * block;
    if (block == 8) {
      reinterpret_cast<int4*>(dst)[0] = make_int4(at(0), at(1), at(2), at(3));
      reinterpret_cast<int4*>(dst)[1] = make_int4(at(4), at(5), at(6), at(7));
    } else {
      for (int t = 0; t < block; ++t) dst[t] = at(t);
    }
  }
}

template <int CPER>
hipError_t launch_cand_topk_kernel(const AttnArgs& a, int block,
                                   const int32_t* limit, int32_t* out,
                                   hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit(
      reinterpret_cast<const void*>(cand_topk_kernel<CPER>),
      kCandTopkSmemBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((cand_topk_kernel<CPER>), dim3(a.B), dim3(512),
                     kCandTopkSmemBytes, s, CSA2_ATTN_HEAD_ARGS(a), a, block,
                     limit, out);
  return hipGetLastError();
}

}  // namespace

int attn_splits(int B, int k) {
  const int n_tiles = (k + kWindow + kTile - 1) / kTile;
  // About one workgroup per compute unit (256 CUs, one workgroup each: its
  // 8 wavefronts take all 512 registers per SIMD lane); with many sequences at
  // least 3 tiles each, to bound the partials' traffic.
  int s = (256 + B - 1) / (B > 0 ? B : 1);
  const int max_s = B >= 16 ? (n_tiles + 2) / 3 : n_tiles;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  // Re-balance so every split has the same number of tiles.
  if (s > kMaxSplits) s = kMaxSplits;
  const int tps = (n_tiles + s - 1) / s;
  return (n_tiles + tps - 1) / tps;
}

size_t attn_workspace(int B, int k) {
  const int s = attn_splits(B, k);
  if (s <= 1) return 0;
  const size_t o = (size_t)B * s * kHeads * 512 * 2;
  const size_t ml = (size_t)B * s * kHeads * 2 * 4;
  return ((o + 255) & ~size_t(255)) + ((ml + 255) & ~size_t(255));
}

namespace {
template <bool FSEL, int CPER>
hipError_t launch_attn_kernel(const AttnArgs& a, unsigned grid, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  const int bytes = FSEL ? kFusedSmemBytes : kSmemBytes;
  hipError_t e = ensure_lds_limit(
      reinterpret_cast<const void*>(attn_kernel<FSEL, CPER>), bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<FSEL, CPER>), dim3(grid), dim3(512), bytes,
                     s, CSA2_ATTN_HEAD_ARGS(a), a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn(const uint8_t* main_codes, const uint8_t* main_scales,
                       int64_t n_cap, const int32_t* topk, int k,
                       const uint16_t* q, const uint8_t* swa,
                       const int32_t* n_swa, int B, float scale,
                       uint16_t* out, void* ws, hipStream_t s,
                       const AttnEpilogue& epi, const FusedSelect* fsel,
                       LaunchMarks* marks) {
  if (B == 0) return hipSuccess;
  AttnArgs a{};
  a.main_codes = main_codes;
  a.main_scales = main_scales;
  a.n_cap = n_cap;
  a.topk = topk;
  a.k = k;
  a.q = q;
  a.swa = swa;
  a.n_swa = n_swa;
  a.scale_log2 = scale * kLog2e;
  a.out = out;
  a.B = B;
  a.n_tiles = (k + kWindow + kTile - 1) / kTile;
  a.n_div = 1;
  a.epi = epi;
  a.splits = attn_splits(B, k);
  a.tiles_per_split = (a.n_tiles + a.splits - 1) / a.splits;
  a.n_main = (k + kTile - 1) / kTile;
  if (a.splits > 1) {
    const size_t o = (size_t)B * a.splits * kHeads * 512 * 2;
    a.part_o = static_cast<uint16_t*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                         ((o + 255) & ~size_t(255)));
  }
  const int groups = (B + 7) / 8;
  const unsigned grid = (unsigned)(8 * groups * a.splits);
  hipError_t e;
  if (fsel) {
    const int C = fsel->n_wg * fsel->kloc;
    if (k > kMaxK || C < 1 || C > kLocalMaxCands) return hipErrorInvalidValue;
    a.lcand = fsel->lcand;
    a.lbound = fsel->lbound;
    a.n_wg = fsel->n_wg;
    a.kloc = fsel->kloc;
    a.keys = fsel->keys;
    a.ld = fsel->ld;
    a.n_entries = fsel->n_entries;
    a.topk_out = fsel->topk_out;
    a.fb_ids = fsel->ids;
    a.fb_n = fsel->n_ids;
    // Candidate pairs per thread.
    if (C <= 1024) e = launch_attn_kernel<true, 2>(a, grid, s);
    else if (C <= 2048) e = launch_attn_kernel<true, 4>(a, grid, s);
    else if (C <= 2560) e = launch_attn_kernel<true, 5>(a, grid, s);
    else e = launch_attn_kernel<true, 8>(a, grid, s);
  } else {
    e = launch_attn_kernel<false, 1>(a, grid, s);
  }
  if (e == hipSuccess && marks) e = marks->mark();
  if (e != hipSuccess || a.splits == 1) return e;
  e = launch_combine<2>(a.part_o, a.part_ml, a.splits, B, out, epi, s);
  if (e == hipSuccess && marks) e = marks->mark();
  return e;
}

hipError_t launch_cand_topk(const uint2* lcand, const uint32_t* lbound,
                            int n_wg, int kloc, const uint32_t* keys,
                            int64_t ld, int64_t n_rows,
                            const int32_t* n_entries, int n_div, int B, int k,
                            int block, const int32_t* limit, int32_t* out,
                            hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int C = n_wg * kloc;
  if (k < 1 || k > kMaxK || C < 1 || C > kCandTopkMax || n_div < 1 ||
      block < 1 || (block == 8 && reinterpret_cast<uintptr_t>(out) % 16))
    return hipErrorInvalidValue;
  AttnArgs a{};
  a.B = B;
  a.k = k;
  a.n_wg = n_wg;
  a.kloc = kloc;
  a.lcand = lcand;
  a.lbound = lbound;
  a.keys = keys;
  a.ld = ld;
  a.n_cap = n_rows;
  a.n_entries = n_entries;
  a.n_div = n_div;
  if (C <= 1024) return launch_cand_topk_kernel<2>(a, block, limit, out, s);
  if (C <= 2048) return launch_cand_topk_kernel<4>(a, block, limit, out, s);
  if (C <= 4096) return launch_cand_topk_kernel<8>(a, block, limit, out, s);
  if (C <= 5120) return launch_cand_topk_kernel<10>(a, block, limit, out, s);
  return launch_cand_topk_kernel<16>(a, block, limit, out, s);
}

}  // namespace csa2
