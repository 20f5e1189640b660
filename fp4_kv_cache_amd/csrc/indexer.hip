// Lightning-indexer scan: I_j = sum_{h<32} w_h * ReLU(q_h . K_j).
//
// Source: "DeepSeek-V4: Towards Highly Efficient Million-Token Context
// Intelligence" (baisen.site), CSA step 2, index-score equation; the same
// form in "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
// (mer.run) section 4.1.  Keys are OCP MXFP4 (E2M1 + E8M0 per 32), section 2
// of the latter page; the pooled block keys of its section 4.3 are bf16.
//
// gfx950 mapping.  One wavefront scores 32 entries per step with the bf16
// matrix core (v_mfma_f32_32x32x16_bf16, 8 issues for the 128-dim dot):
// A = the 32 query heads (held in VGPRs for the whole scan), B = 32 keys
// dequantised in registers from their FP4 codes with the packed
// scale-convert (E2M1 x 2^e is exact in bf16, so every product is exact and
// only the float32 accumulation rounds).  The dot product does not depend on
// the order of its terms, so lane half h of the wave takes dims
// 64h .. 64h+63 of its key: each lane streams one contiguous 32-byte run of
// codes (two 16-byte loads) and the query is permuted the same way.  The
// accumulator comes out head-major (16 heads per lane); ReLU, the head
// weights and the head sum are applied per lane and the two lane halves are
// folded with one cross-half swap.  HBM traffic per entry: 64 + 4 bytes
// read, 4 bytes of score written.
//
// FP4 query ("DeepSeek-V4.1-Flash, 2. Architecture" course notes, 2.4.4:
// V4 trains the indexer query and key for FP4, OCP MXFP4, so that scoring
// itself runs on FP4; the mer.run page, section 5, says the same).  With
// the query also in MXFP4, an MXFP4 tile is two issues of the gfx950 scaled
// matrix op v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 x E2M1 with one E8M0
// scale per 32 values on each side) straight from the loaded code bytes:
// no conversion at all.  Operand layout of that op: lane l holds row (or
// column) l % 32 and the 32 consecutive K values 32*(l/32) .. +31, two per
// byte, low nibble first -- exactly the stored order -- and the scale byte
// picked by op_sel.  Lane half h feeds dims 64h .. 64h+31 to the first
// issue and 64h+32 .. 64h+63 to the second (the query in the same order),
// so its 32 code bytes are the two operands as loaded and its scale bytes
// are 2h and 2h+1.  Every product is exact; the sums are float32.  The
// bf16 block keys take the query dequantised to bf16, which is exact.
//
// Selection keys: with KEYS the scores are written as order-preserving
// uint32 keys, and either each 32-row tile's largest key (the top-k stage
// then reads only the tiles that can hold a winner) or, in the decode path,
// each group's own top entries and a bound (local candidates, below), from
// which the attention workgroups select the top-k themselves.  There the
// sequence's query is read once per workgroup and staged in LDS, and
// nothing the first key loads do not need is read before them.
#include "common.h"
#include "internal.h"
#include "select.h"

#include <algorithm>

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kTilesPerWave = 8;    // 32-entry tiles per wavefront

// Raw key data one lane holds for one 32-entry tile.
template <int KEYFMT> struct RawKey;
template <> struct RawKey<0> {       // MXFP4: 32 code bytes + 2 scale bytes
  u32x4 c0, c1;
  uint32_t sc;
};
template <> struct RawKey<1> {       // bf16: 64 dims = 128 bytes
  u32x4 v[8];
};

// Loads are unconditional (the caller clamps `row` to a row that exists), so
// no load sits inside a branch and the compiler can keep several tiles of
// loads in flight with exact wait counts.  `codes`/`scales` point at the
// sequence's first row and `row` is the row within it: byte offsets stay
// below 2^32 (n_cap <= 2^24), one uniform base plus a 32-bit lane offset.
// HALF_SCALES (scaled matrix op): only this lane half's two scale bytes
// (2*half, 2*half+1), as bits 0-15, so the op reads the loaded register as
// it is and nothing waits on the load before the op itself.
template <int KEYFMT, bool HALF_SCALES>
__device__ __forceinline__ void load_key(RawKey<0>& r, const void* codes,
                                         const uint8_t* scales, uint32_t row,
                                         int half) {
  const u32x4* p = reinterpret_cast<const u32x4*>(
      static_cast<const uint8_t*>(codes) + (row * 64u + 32u * half));
  r.c0 = p[0];
  r.c1 = p[1];
  if constexpr (HALF_SCALES)
    r.sc = *reinterpret_cast<const uint16_t*>(scales + (row * 4u + 2u * half));
  else
    r.sc = *reinterpret_cast<const uint32_t*>(scales + row * 4u);
}

template <int KEYFMT, bool HALF_SCALES>
__device__ __forceinline__ void load_key(RawKey<1>& r, const void* codes,
                                         const uint8_t*, uint32_t row,
                                         int half) {
  const u32x4* p = reinterpret_cast<const u32x4*>(
      static_cast<const uint8_t*>(codes) + (row * 256u + 128u * half));
#pragma unroll
  for (int s = 0; s < 8; ++s) r.v[s] = p[s];
}

// B operand of step s: 8 dims 64h + 8s .. +7 of this lane's key, as bf16.
template <int KEYFMT>
__device__ __forceinline__ bf16x8 key_operand(const RawKey<KEYFMT>& r, int s,
                                              int half);

template <>
__device__ __forceinline__ bf16x8 key_operand<0>(const RawKey<0>& r, int s,
                                                 int half) {
  const uint32_t cw = s < 4 ? r.c0[s] : r.c1[s - 4];
  const uint32_t sbyte = (r.sc >> (8 * (2 * half + (s >> 2)))) & 0xFFu;
  const float sf = e8m0_to_f32(sbyte);
  u32x4 o;
  o[0] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 0));
  o[1] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 1));
  o[2] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 2));
  o[3] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 3));
  return bits_to_bf8(o);
}

template <>
__device__ __forceinline__ bf16x8 key_operand<1>(const RawKey<1>& r, int s,
                                                 int) {
  return bits_to_bf8(r.v[s]);
}

// FP4 operand of the scaled matrix op: 32 E2M1 values in the low 16 bytes
// (the upper half of the register group is not read for FP4).
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x8 fp4_operand(u32x4 v) {
  i32x8 o;
  o[0] = (int32_t)v[0]; o[1] = (int32_t)v[1];
  o[2] = (int32_t)v[2]; o[3] = (int32_t)v[3];
  o[4] = 0; o[5] = 0; o[6] = 0; o[7] = 0;
  return o;
}
constexpr int kFmtFp4 = 4;          // E2M1 in the op's format fields

// Tiles of loads kept in flight ahead of the matrix work (the scaled-op
// path does little per tile, so it keeps one more).  The bf16 block keys
// (8 KB per wavefront tile) keep two as well, at 2 wavefronts per SIMD
// instead of 4: the 8 x 131,072-block scan's decode step measured 122.8
// against 125.0 us with one.
template <int KEYFMT, bool SCALED> struct Depth {
  static constexpr int value = SCALED ? 3 : 2;
};

// Entry ids of rows id0 .. id0+PER-1 of a local-candidate group: the rows
// themselves, or with candidate ids the entries they name (rows past the end
// read the last row; their keys are 0, so they are never kept).
template <bool CAND, int PER>
__device__ __forceinline__ void entry_ids(const int32_t* cand, int b,
                                          int64_t n_rows, uint32_t id0,
                                          uint32_t (&eid)[PER]) {
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if constexpr (CAND) {
      const int64_t i = (int64_t)id0 + j;
      eid[j] = (uint32_t)cand[(int64_t)b * n_rows + (i < n_rows ? i : n_rows - 1)];
    } else {
      eid[j] = id0 + j;
    }
  }
}

// Selection keys of rows i0 .. i0+PER-1 of sequence b (i0 a multiple of
// PER), as 16-byte stores into the key row, which is padded to a multiple of
// 32 entries: rows past n_rows inside the padding take their key, 0
// (invalid); runs past the padding are not written.
template <int PER>
__device__ __forceinline__ void store_keys(float* scores, int b,
                                           int64_t n_rows, int64_t i0,
                                           const uint32_t (&kk)[PER]) {
  static_assert(PER % 4 == 0 && 32 % PER == 0, "whole 16-byte runs");
  const int64_t ld32 = (n_rows + 31) & ~(int64_t)31;
  if (i0 >= ld32) return;
  uint4* dst = reinterpret_cast<uint4*>(
      reinterpret_cast<uint32_t*>(scores) + (int64_t)b * ld32 + i0);
#pragma unroll
  for (int j = 0; j < PER; j += 4)
    dst[j / 4] = make_uint4(kk[j], kk[j + 1], kk[j + 2], kk[j + 3]);
}

// KEYS: write selection keys (see score_key) instead of float scores, and
// each 32-row tile's largest key to tmax[B][ceil(n_rows/32)]; with `bmax`
// also each 8-row block's largest key to bmax[B][round32(nb)] (nb =
// ceil(n_rows/8)) and each 256-row group's (a wavefront's rows) to
// btmax[B][ceil(nb/32)].
// QFP4: the query is MXFP4 planes (codes q[B][32][64], scales
// q_scales[B][32][4]) instead of bf16 q[B][32][128].  BLK (with KEYS):
// the block maxima are written too.
// LOCAL (with KEYS): instead of tile maxima, each group of rows also keeps
// its own local top-kloc entries as (key, id) pairs, in row order, in
// lcand[B][groups][kloc] (key 0 / id -1 padding; the id is the row, or with
// CAND the entry the row names, so ids run in row order whenever the
// candidate ids ascend), and
// in lbound[B][groups] a key at or above every valid entry it left out (0
// when it left none out).  The union of every group's pairs then holds the
// row's top-k whenever the k-th largest pair key is above every bound: a
// selection over the small union is exact under that test.  A group is a
// wavefront's rows (LOCAL == 1: no barrier, each wavefront selects alone)
// or a workgroup's (LOCAL == 2: larger groups for long rows).
template <int KEYFMT, bool KEYS, bool QFP4, bool BLK = false, bool CAND = false,
          int TPW = kTilesPerWave, int LOCAL = 0>
// The arguments a wavefront needs before its first key loads (the key
// planes, the query, the weights, the candidate ids and the row count) come
// first: the first 14 dwords are preloaded into scalar registers at
// dispatch.  The entry count is read after the first key loads are issued.
__global__ __launch_bounds__(256) void indexer_kernel(
    const void* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    int64_t n_cap, const void* __restrict__ q_in,
    const float* __restrict__ w, const int32_t* __restrict__ cand,
    int64_t n_rows, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q_scales, float* __restrict__ scores,
    uint32_t* __restrict__ tmax, uint32_t* __restrict__ bmax,
    uint32_t* __restrict__ btmax, int n_div, uint2* __restrict__ lcand,
    uint32_t* __restrict__ lbound, int kloc) {
  constexpr bool kScaledOp = QFP4 && KEYFMT == 0;
  constexpr int D = Depth<KEYFMT, kScaledOp>::value;
  constexpr int T = TPW;
  static_assert(LOCAL == 0 || (KEYS && !BLK && (KEYFMT == 0 || !CAND)),
                "local candidates: selection keys, no block maxima");
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int64_t base =
      ((int64_t)blockIdx.x * kWaves + wave) * (T * 32);
  // The local selection: the workgroup's keys in id order, then its
  // selection histograms (zeroed here; the selection's first barrier comes
  // long after).  A wavefront past the rows still takes part (its keys are
  // all invalid), so no wavefront leaves before the selection's barriers.
  extern __shared__ __align__(16) uint32_t lsm[];
  uint32_t* kl = lsm;
  SelSmem<256, 256>& lss =
      *reinterpret_cast<SelSmem<256, 256>*>(lsm + kWaves * T * 32);
  if constexpr (LOCAL == 1) {
    // Each wavefront clears its own histogram (its LDS operations take
    // effect in order, so no barrier is needed before its selection).
    reinterpret_cast<int4*>(lss.hist[wave])[lane] = make_int4(0, 0, 0, 0);
  } else if constexpr (LOCAL == 2) {
    for (int i = threadIdx.x; i < kWaves * 256; i += 256)
      (&lss.hist[0][0])[i] = 0;
  } else {
    if (base >= n_rows) return;                // wave-uniform; no barriers
  }
  // Valid rows: n_entries[b], or for bf16 block keys ceil(n_entries[b] /
  // n_div) (rows are blocks of n_div entries; 32-bit unsigned, exact for
  // these ranges), never past the cache.  The MXFP4 scan carries no
  // division: it would sit before every wavefront's first load.
  const void* seq_codes = static_cast<const uint8_t*>(k_codes) +
                          (int64_t)b * n_cap * (KEYFMT == 0 ? 64 : 256);
  const uint8_t* seq_scales =
      KEYFMT == 0 ? k_scales + (int64_t)b * n_cap * 4 : nullptr;
  const int64_t nt64 = base < n_rows ? (n_rows - base + 31) >> 5 : 0;
  const int nt = nt64 < T ? (int)nt64 : T;

  // Row (within the sequence) of every tile position this lane will read,
  // with validity; invalid rows are clamped to row 0.  Candidate ids are
  // loaded first, all in one round (one wait, not one per tile); without
  // them the row of tile t is base + 32t + col, formed where it is used
  // (8 registers fewer).
  uint32_t crow_v[CAND ? T : 1];
  uint32_t vmask = 0;
  if constexpr (CAND) {
    int32_t cv[T];
    const int32_t* crow = cand + (int64_t)b * n_rows;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t i = base + 32 * t + col;
      cv[t] = crow[i < n_rows ? i : n_rows - 1];
    }
    // Rows to load are bounded by the cache (so the loads do not wait for
    // the entry count); validity (below) also needs the id below the count.
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t i = base + 32 * t + col;
      const int64_t e = cv[t];
      const bool in = (i < n_rows) & (e >= 0) & (e < n_cap);
      vmask |= (in ? 1u : 0u) << t;
      crow_v[t] = in ? (uint32_t)e : 0u;
    }
  }
  // The first tiles' rows are bounded by the cache alone, so their loads
  // do not wait for the sequence's entry count (their scores are masked
  // by it like every other tile's).
  const uint32_t r0 = (uint32_t)base + (uint32_t)col;
  const uint32_t lim_rows = (uint32_t)n_rows;
  auto row_pf = [&](int t) -> uint32_t {
    if constexpr (CAND) return crow_v[t];
    else return r0 + 32u * t < lim_rows ? r0 + 32u * t : 0u;
  };

  // A operand: head `col`, dims 64*half + 8*s .. +7 for step s (bf16), or
  // the head's MXFP4 codes for dims 64*half .. +63 and its two scale bytes
  // for them in bits 0-15 (scaled op).
  bf16x8 qa[kScaledOp ? 1 : 8];
  RawKey<0> q4;
  if constexpr (QFP4) {
    // The codes now; the scales (their pointer is not a preloaded
    // argument) after the first key loads.
    const int64_t head = (int64_t)b * kIdxHeads + col;
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint8_t*>(q_in) + head * 64 + 32 * half);
    q4.c0 = qp[0];
    q4.c1 = qp[1];
  }
  // bf16 query with local candidates (no wavefront leaves early): the
  // workgroup reads the sequence's 8 KB query and 32 weights once,
  // coalesced (thread i: 16-byte pieces i and i + 256), and stages them in
  // LDS (head rows padded by 16 bytes); the first tiles' key loads are
  // issued before the barrier, so they are in flight meanwhile.  Read per
  // wavefront, the query was 32 KB of requests per workgroup ahead of the
  // first key loads.
  constexpr bool kStageQ = !QFP4 && LOCAL != 0;
  __shared__ __align__(16) u32x4 q_lds[kStageQ ? kIdxHeads * 17 : 1];
  __shared__ float w_lds[kStageQ ? kIdxHeads : 1];
  u32x4 qv0, qv1;
  float wv = 0.0f;
  if constexpr (kStageQ) {
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(q_in) + (int64_t)b * kIdxHeads * kIdxDim);
    qv0 = qsrc[threadIdx.x];
    qv1 = qsrc[threadIdx.x + 256];
    if (threadIdx.x < kIdxHeads) wv = w[b * kIdxHeads + threadIdx.x];
  } else if constexpr (!QFP4) {
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
        static_cast<const uint16_t*>(q_in) +
        ((int64_t)b * kIdxHeads + col) * kIdxDim + 64 * half);
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[s] = qrow[s];
  }
  RawKey<KEYFMT> buf[D + 1];
#pragma unroll
  for (int t = 0; t < D; ++t)
    load_key<KEYFMT, kScaledOp>(buf[t], seq_codes, seq_scales, row_pf(t), half);
  // The entry count, and everything that needs it, comes after the first
  // key loads are issued (its pointer is not among the preloaded arguments,
  // so its load would otherwise wait for an argument-line miss first).
  __builtin_amdgcn_sched_barrier(0);
  // Valid rows: n_entries[b], or for bf16 block keys ceil(n_entries[b] /
  // n_div) (rows are blocks of n_div entries; 32-bit unsigned, exact for
  // these ranges), never past the cache.
  if constexpr (QFP4) {
    const int64_t head = (int64_t)b * kIdxHeads + col;
    q4.sc = *reinterpret_cast<const uint32_t*>(q_scales + head * 4);
    if constexpr (kScaledOp) {
      q4.sc >>= 16 * half;
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qa[s] = key_operand<0>(q4, s, half);
    }
  }
  const int32_t ne = n_entries[b];
  int64_t n = ne <= 0 ? 0 : (int64_t)ne;
  if constexpr (KEYFMT == 1)
    if (ne > 0 && n_div > 1)
      n = (int64_t)(((uint32_t)ne + (uint32_t)n_div - 1u) / (uint32_t)n_div);
  n = n > n_cap ? n_cap : n;
  if constexpr (CAND) {
    // A named row is valid below the entry count (n <= n_cap).
#pragma unroll
    for (int t = 0; t < T; ++t)
      if ((int64_t)crow_v[t] >= n) vmask &= ~(1u << t);
  }
  // Plain rows: valid below lim = min(n_rows, n); base < 2^24.
  const uint32_t lim = (uint32_t)(n_rows < n ? n_rows : n);
  auto row_of = [&](int t) -> uint32_t {
    if constexpr (CAND) return crow_v[t];
    else return r0 + 32u * t < lim ? r0 + 32u * t : 0u;
  };
  auto valid = [&](int t) -> bool {
    if constexpr (CAND) return (vmask >> t) & 1u;
    else return r0 + 32u * t < lim;
  };
  // Weights of the 16 output rows this lane holds: head 8a + 4*half + r.
  float wr[16];
  if constexpr (kStageQ) {
    const int i0 = threadIdx.x, i1 = threadIdx.x + 256;
    q_lds[(i0 >> 4) * 17 + (i0 & 15)] = qv0;
    q_lds[(i1 >> 4) * 17 + (i1 & 15)] = qv1;
    if (threadIdx.x < kIdxHeads) w_lds[threadIdx.x] = wv;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[s] = bits_to_bf8(q_lds[col * 17 + 8 * half + s]);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[4 * a + r] = w_lds[8 * a + 4 * half + r];
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        wr[4 * a + r] = w[b * kIdxHeads + 8 * a + 4 * half + r];
  }
  float total[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (t + D < T)
      load_key<KEYFMT, kScaledOp>(buf[(t + D) % (D + 1)], seq_codes,
                                  seq_scales, row_of(t + D), half);
    // MXFP4 keys: no branch around the tile -- a conditional block would
    // let the compiler sink this tile's loads into it (and serialise them);
    // tiles past the end compute on clamped rows and are masked out.  The
    // bf16 block keys (one tile of loads ahead) keep the per-tile test,
    // which schedules better there.
    if (KEYFMT == 0 || (t < nt && base + 32 * t < (CAND ? n_rows : n))) {
      const RawKey<KEYFMT>& cur = buf[t % (D + 1)];
      f32x16 acc = {};
      if constexpr (kScaledOp) {
        const int32_t ks = (int32_t)cur.sc;   // bytes 2*half, 2*half+1
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fp4_operand(q4.c0), fp4_operand(cur.c0), acc, kFmtFp4, kFmtFp4,
            0, (int32_t)q4.sc, 0, ks);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fp4_operand(q4.c1), fp4_operand(cur.c1), acc, kFmtFp4, kFmtFp4,
            1, (int32_t)q4.sc, 1, ks);
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              qa[s], key_operand<KEYFMT>(cur, s, half), acc, 0, 0, 0);
      }
      // ReLU as an integer max on the float bits (negatives and -0 go to
      // +0; the dots are finite), weights, and the head sum in two chains.
      float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        p0 += wr[j] * __int_as_float(max(__float_as_int(acc[j]), 0));
        p1 += wr[j + 1] * __int_as_float(max(__float_as_int(acc[j + 1]), 0));
      }
      // Fold the lane halves (the two halves hold different heads of the
      // same entry): the swap gives every lane both halves' partial head
      // sums, added in the same order.
      const auto hv = __builtin_amdgcn_permlane32_swap(
          __float_as_uint(p0 + p1), __float_as_uint(p0 + p1), false, false);
      const float sum = __uint_as_float(hv[0]) + __uint_as_float(hv[1]);
      total[t] = valid(t) ? sum : -__builtin_inff();
    } else {
      total[t] = -__builtin_inff();
    }
    // Local candidates: the tile's keys go to the wavefront's stretch of
    // LDS at once (LDS writes count apart from the loads' wait counts), so
    // no score stays live across the loop.
    if constexpr (LOCAL != 0)
      if (half == 0) kl[wave * T * 32 + 32 * t + col] = score_key(total[t]);
  }
  // Stores after the loop keep the loads' wait counts static.
  static_assert(!BLK || T * 32 == 256, "a wavefront's rows are one "
                "32-block group of the block maxima");
  uint32_t wmax = 0u;
#pragma unroll
  for (int t = 0; t < (LOCAL == 0 ? T : 0); ++t) {
    if (t >= nt) break;
    const int64_t i = base + 32 * t + col;
    if constexpr (KEYS) {
      // Selection keys (rows padded to a multiple of 32 entries, so whole
      // tiles can be read as aligned 16-byte vectors), and each tile's
      // largest key (both lane halves hold the same 32 entries) by an
      // integer wavefront maximum.
      const uint32_t key = score_key(total[t]);
      const int64_t ld32 = (n_rows + 31) & ~(int64_t)31;
      if (half == 0 && i < n_rows)
        reinterpret_cast<uint32_t*>(scores)[(int64_t)b * ld32 + i] = key;
      // The tile maximum by the DPP max network (as wave_max_u32); after
      // its first three steps lane 8j+7 holds the largest key of entries
      // 8j .. 8j+7: the block maximum of the hierarchical pool.
      uint32_t m = dpp_max<0x111, 0xf>(key);
      m = dpp_max<0x112, 0xf>(m);
      m = dpp_max<0x114, 0xf>(m);
      if (BLK && half == 0 && (col & 7) == 7) {
        const int64_t nbs = (n_rows + 7) >> 3;
        const int64_t blk = i >> 3;
        if (blk < nbs) bmax[(int64_t)b * ((nbs + 31) & ~(int64_t)31) + blk] = m;
      }
      m = dpp_max<0x118, 0xf>(m);
      m = dpp_max<0x142, 0xa>(m);
      m = dpp_max<0x143, 0xc>(m);
      const uint32_t mx = (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
      if (LOCAL == 0 && lane == 0)
        tmax[(int64_t)b * ((n_rows + 31) >> 5) + ((base >> 5) + t)] = mx;
      if constexpr (BLK) wmax = max(wmax, mx);
    } else {
      if (half == 0 && i < n_rows) scores[(int64_t)b * n_rows + i] = total[t];
    }
  }
  if (BLK && lane == 0) {
    const int64_t nbt = (((n_rows + 7) >> 3) + 31) >> 5;
    btmax[(int64_t)b * nbt + (base >> 8)] = wmax;
  }
  if constexpr (LOCAL == 1) {
    // Tiles past the rows hold invalid keys.  Lane i takes the wavefront's
    // rows PER*i .. PER*i+PER-1 (position order is id order), read back
    // from the wavefront's own stretch of LDS.
    for (int t = nt; t < T; ++t)
      if (half == 0) kl[wave * T * 32 + 32 * t + col] = 0u;
    constexpr int PER = T / 2;
    uint32_t kk[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) kk[j] = kl[wave * T * 32 + lane * PER + j];
    store_keys<PER>(scores, b, n_rows, base + lane * PER, kk);
    const uint32_t id0 = (uint32_t)(base + lane * PER);
    uint32_t eid[PER];
    entry_ids<CAND, PER>(cand, b, n_rows, id0, eid);
    const WaveCut r = wave_cut<PER>(kk, kloc, lss.hist[wave]);
    const int64_t grp = ((int64_t)b * gridDim.x + blockIdx.x) * kWaves + wave;
    uint2* co = lcand + grp * kloc;
    int p = r.pos;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (r.mask & (1u << j)) co[p++] = make_uint2(kk[j], eid[j]);
    for (int q = r.total + lane; q < kloc; q += 64)
      co[q] = make_uint2(0u, 0xFFFFFFFFu);
    if (lane == 0) lbound[grp] = r.bound;
  }
  if constexpr (LOCAL == 2) {
    // Tiles past the rows hold invalid keys.
    for (int t = nt; t < T; ++t)
      if (half == 0) kl[wave * T * 32 + 32 * t + col] = 0u;
    __syncthreads();
    // Thread i takes entries PER*i .. PER*i+PER-1 of the workgroup, so the
    // selection's position order is id order.
    constexpr int PER = T / 2;
    const int tid = threadIdx.x;
    uint32_t kk[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) kk[j] = kl[tid * PER + j];
    store_keys<PER>(scores, b, n_rows,
                    (int64_t)blockIdx.x * (kWaves * T * 32) + tid * PER, kk);
    const uint32_t id0 = (uint32_t)(blockIdx.x * (kWaves * T * 32) + tid * PER);
    uint32_t eid[PER];
    entry_ids<CAND, PER>(cand, b, n_rows, id0, eid);
    const SelResult r = block_select<256, PER, 256>(kk, kloc, lss);
    const int64_t wg = (int64_t)b * gridDim.x + blockIdx.x;
    uint2* co = lcand + wg * kloc;
    int p = r.pos;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (r.mask & (1u << j)) co[p++] = make_uint2(kk[j], eid[j]);
    for (int q = r.total + tid; q < kloc; q += 256)
      co[q] = make_uint2(0u, 0xFFFFFFFFu);
    // Every valid entry left out is <= thr (the selection ends on the k-th
    // key's own value, or takes exactly the keys >= thr).
    if (tid == 0) lbound[wg] = r.nval > kloc ? r.thr : 0u;
  }
}

}  // namespace

namespace {
// A plain MXFP4-key scan with the bf16 query takes 16 tiles per wavefront
// once 8 would need two or more generations of wavefronts (4 per SIMD on
// 256 CUs): each wavefront loads the 8 KB query, and there the dispatcher's
// balancing no longer needs the shorter wavefronts (64 x 131,072 entries:
// 112.9 against 121.1 us; 4 x 524,288: 30.7 against 32.0 us).  A single
// generation (32 x 32,768) keeps 8; the MXFP4 query (2 KB) gains nothing.
constexpr int64_t kLongScanWaves = 2 * 4096;

template <int KEYFMT, bool KEYS, bool QFP4>
void launch_one(int B, hipStream_t s, const void* k_codes,
                const uint8_t* k_scales, int64_t n_cap,
                const int32_t* n_entries, const int32_t* cand, int64_t n_rows,
                const IndexQuery& iq, float* scores, uint32_t* tmax,
                uint32_t* bmax, uint32_t* btmax, int n_div) {
  const auto grid_for = [&](int tpw) {
    const int64_t epb = (int64_t)kWaves * tpw * 32;
    return dim3((unsigned)((n_rows + epb - 1) / epb), (unsigned)B);
  };
  const dim3 grid = grid_for(kTilesPerWave);
  const int64_t waves = (int64_t)grid.x * grid.y * kWaves;
  if (KEYFMT == 0 && !QFP4 && !bmax && !cand && waves >= kLongScanWaves)
    hipLaunchKernelGGL((indexer_kernel<0, KEYS, false, false, false, 16>),
                       grid_for(16), dim3(256), 0, s, k_codes, k_scales,
                       n_cap, iq.q, iq.w, cand, n_rows, n_entries,
                       iq.q_scales, scores, tmax, bmax, btmax, n_div, nullptr,
                       nullptr, 0);
  else if (KEYS && KEYFMT == 0 && !QFP4 && bmax)
    hipLaunchKernelGGL((indexer_kernel<0, true, false, true>), grid,
                       dim3(256), 0, s, k_codes, k_scales, n_cap, iq.q,
                       iq.w, cand, n_rows, n_entries, iq.q_scales, scores, tmax,
                       bmax, btmax, n_div, nullptr, nullptr, 0);
  else if (cand)
    hipLaunchKernelGGL((indexer_kernel<KEYFMT, KEYS, QFP4, false, true>),
                       grid, dim3(256), 0, s, k_codes, k_scales, n_cap,
                       iq.q, iq.w, cand, n_rows, n_entries, iq.q_scales,
                       scores, tmax, bmax, btmax, n_div, nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL((indexer_kernel<KEYFMT, KEYS, QFP4>), grid, dim3(256),
                       0, s, k_codes, k_scales, n_cap, iq.q, iq.w,
                       cand, n_rows, n_entries, iq.q_scales, scores, tmax, bmax,
                       btmax, n_div, nullptr, nullptr, 0);
}
template <int KEYFMT, bool KEYS>
void launch_q(int B, hipStream_t s, const void* k_codes,
              const uint8_t* k_scales, int64_t n_cap, const int32_t* n_entries,
              const int32_t* cand, int64_t n_rows, const IndexQuery& iq,
              float* scores, uint32_t* tmax, uint32_t* bmax,
              uint32_t* btmax, int n_div) {
  if (iq.q_scales)
    launch_one<KEYFMT, KEYS, true>(B, s, k_codes, k_scales, n_cap,
                                   n_entries, cand, n_rows, iq, scores, tmax,
                                   bmax, btmax, n_div);
  else
    launch_one<KEYFMT, KEYS, false>(B, s, k_codes, k_scales, n_cap,
                                    n_entries, cand, n_rows, iq, scores, tmax,
                                    bmax, btmax, n_div);
}
template <int KF, bool QFP4, int T, int LOCAL, bool CAND>
hipError_t launch_local(int B, hipStream_t s, const void* k_codes,
                        const uint8_t* k_scales, int64_t n_cap,
                        const int32_t* n_entries, const int32_t* cand,
                        int64_t n_rows, const IndexQuery& iq, uint32_t* keys,
                        const LocalPlan& lp, uint2* lcand, uint32_t* lbound,
                        int n_div) {
  const int smem = (kWaves * T * 32 + kWaves * 256 + 16) * 4;
  const int64_t epb = (int64_t)kWaves * T * 32;
  hipLaunchKernelGGL(
      (indexer_kernel<KF, true, QFP4, false, CAND, T, LOCAL>),
      dim3((unsigned)((n_rows + epb - 1) / epb), (unsigned)B), dim3(256),
      smem, s, k_codes, k_scales, n_cap, iq.q, iq.w, cand, n_rows, n_entries,
      iq.q_scales, reinterpret_cast<float*>(keys), nullptr, nullptr,
      nullptr, n_div, lcand, lbound, lp.kloc);
  return hipGetLastError();
}
}  // namespace

LocalPlan local_plan(int B, int64_t n_cap, int k, bool qfp4, bool cand,
                     int max_cands) {
  LocalPlan lp;
  if (B < 1 || n_cap < 1 || k < 1) return lp;
  // The same wavefront length as the plain scan (see kLongScanWaves); a
  // scan of candidate rows keeps 8 tiles.
  const int64_t per8 = (int64_t)kWaves * 8 * 32;
  const int64_t waves8 = ((n_cap + per8 - 1) / per8) * (int64_t)B * kWaves;
  lp.tpw = (!qfp4 && !cand && waves8 >= kLongScanWaves) ? 16 : 8;
  const int64_t epb = (int64_t)kWaves * lp.tpw * 32;      // rows per workgroup
  const int64_t n_wg = (n_cap + epb - 1) / epb;
  // Groups of one wavefront's rows while every group can keep 20 pairs (a
  // group expects k * rows / n of the row's winners: 4 for 512 of 32,768
  // in 256 rows, so 20 are exceeded with probability ~1e-9 on independent
  // scores), else groups of a workgroup's rows keeping 16 or more (40 when
  // there is room: 2,048 of 131,072 blocks in 1,024 rows expect 16, and
  // exceed 40 with probability ~3e-8).
  for (int per_wave = 1; per_wave >= 0; --per_wave) {
    const int64_t groups = per_wave ? n_wg * kWaves : n_wg;
    const int64_t rows = per_wave ? epb / kWaves : epb;
    const int64_t kmin = per_wave ? 20 : 16;
    int64_t kl = std::max<int64_t>(per_wave ? 20 : 40,
                                   (2 * (int64_t)k + groups - 1) / groups);
    kl = std::min<int64_t>(kl, rows);
    kl = std::min<int64_t>(kl, max_cands / groups);
    if (kl < std::min<int64_t>(kmin, rows) || kl * groups < 2 * (int64_t)k)
      continue;
    lp.ok = true;
    lp.per_wave = per_wave != 0;
    lp.n_wg = (int)groups;
    lp.kloc = (int)kl;
    return lp;
  }
  return lp;
}

hipError_t launch_indexer_local(const uint8_t* k_codes,
                                const uint8_t* k_scales, int64_t n_cap,
                                const int32_t* n_entries,
                                const IndexQuery& iq, int B, uint32_t* keys,
                                const LocalPlan& lp, uint2* lcand,
                                uint32_t* lbound, hipStream_t s,
                                const int32_t* cand, int64_t n_rows,
                                int keyfmt, int n_div) {
  if (B == 0) return hipSuccess;
  if (!lp.ok) return hipErrorInvalidValue;
  const bool q4 = iq.q_scales != nullptr;
  const bool c = cand != nullptr;
  if (!c) n_rows = n_cap;
  if (n_rows < 1) return hipErrorInvalidValue;
  if (keyfmt == 1) {
    // bf16 block keys: rows are blocks of n_div entries, 8 tiles.
    if (c || lp.tpw != 8) return hipErrorInvalidValue;
#define CSA2_LOCAL_B(Q, L)                                                   \
    if (q4 == Q && (lp.per_wave ? 1 : 2) == L)                               \
      return launch_local<1, Q, 8, L, false>(B, s, k_codes, nullptr, n_cap,  \
                                             n_entries, nullptr, n_rows, iq,  \
                                             keys, lp, lcand, lbound, n_div);
    CSA2_LOCAL_B(false, 1)
    CSA2_LOCAL_B(false, 2)
    CSA2_LOCAL_B(true, 1)
    CSA2_LOCAL_B(true, 2)
#undef CSA2_LOCAL_B
    return hipErrorInvalidValue;
  }
#define CSA2_LOCAL(Q, T, L, C)                                               \
  if (q4 == Q && lp.tpw == T && (lp.per_wave ? 1 : 2) == L && c == C)        \
    return launch_local<0, Q, T, L, C>(B, s, k_codes, k_scales, n_cap,       \
                                       n_entries, cand, n_rows, iq, keys, lp, \
                                       lcand, lbound, 1);
  CSA2_LOCAL(true, 8, 1, false)
  CSA2_LOCAL(true, 8, 2, false)
  CSA2_LOCAL(false, 8, 1, false)
  CSA2_LOCAL(false, 8, 2, false)
  CSA2_LOCAL(false, 16, 1, false)
  CSA2_LOCAL(false, 16, 2, false)
  CSA2_LOCAL(true, 8, 1, true)
  CSA2_LOCAL(true, 8, 2, true)
  CSA2_LOCAL(false, 8, 1, true)
  CSA2_LOCAL(false, 8, 2, true)
#undef CSA2_LOCAL
  return hipErrorInvalidValue;
}

hipError_t launch_indexer(int keyfmt, const void* k_codes,
                          const uint8_t* k_scales, int64_t n_cap,
                          const int32_t* n_entries, const int32_t* cand,
                          int64_t n_rows, const IndexQuery& iq, int B,
                          float* scores, hipStream_t s, uint32_t* tmax,
                          uint32_t* bmax, uint32_t* btmax, int n_div) {
  if (n_rows == 0 || B == 0) return hipSuccess;
  if (n_div < 1 || (n_div > 1 && keyfmt != 1)) return hipErrorInvalidValue;
  // Block maxima: MXFP4 keys, bf16 query, all rows.
  if (bmax && (!tmax || cand || !btmax || keyfmt != 0 || iq.q_scales))
    return hipErrorInvalidValue;
  if (keyfmt == 0 && tmax)
    launch_q<0, true>(B, s, k_codes, k_scales, n_cap, n_entries, cand,
                      n_rows, iq, scores, tmax, bmax, btmax, n_div);
  else if (keyfmt == 0)
    launch_q<0, false>(B, s, k_codes, k_scales, n_cap, n_entries, cand,
                       n_rows, iq, scores, tmax, bmax, btmax, n_div);
  else if (tmax)
    launch_q<1, true>(B, s, k_codes, k_scales, n_cap, n_entries, cand,
                      n_rows, iq, scores, tmax, bmax, btmax, n_div);
  else
    launch_q<1, false>(B, s, k_codes, k_scales, n_cap, n_entries, cand,
                       n_rows, iq, scores, tmax, bmax, btmax, n_div);
  return hipGetLastError();
}

}  // namespace csa2
