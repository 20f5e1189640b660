// Host-side launchers behind the C ABI (enqueue only; arguments validated
// by the caller in api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// pack.hip
hipError_t launch_pack_main(const float* src, int64_t n, uint8_t* codes,
                            uint8_t* scales, hipStream_t s);
hipError_t launch_pack_idx(const float* src, int64_t n, uint8_t* codes,
                           uint8_t* scales, hipStream_t s);
hipError_t launch_pack_swa(const float* src, int64_t n, uint8_t* codes,
                           hipStream_t s);
hipError_t launch_unpack(int fmt, const uint8_t* codes, const uint8_t* scales,
                         int64_t n, float* dst, hipStream_t s);
hipError_t launch_block_keys(const uint8_t* codes, const uint8_t* scales,
                             int64_t n_cap, const int32_t* n_entries, int B,
                             int block, uint16_t* keys, hipStream_t s);

// indexer.hip
// Scores rows (all n_rows, or the n_rows candidate ids `cand`) into float
// scores[B][n_rows].  With `tmax` (the decode path) it writes selection keys
// (score_key, as uint32) instead, rows padded to a multiple of 32 entries
// (scores[B][round_up(n_rows, 32)]), and each 32-row tile's largest key into
// tmax[B][ceil(n_rows/32)].  A row is valid below n_entries[b], or for bf16
// block keys below ceil(n_entries[b] / n_div) (rows are blocks of n_div
// entries; n_div > 1 only with those keys).  With `bmax` (and `btmax`; all rows, no
// candidates) also the 8-row block maxima bmax[B][round_up(nb, 32)], nb =
// ceil(n_rows/8), and their 32-block maxima btmax[B][ceil(nb/32)].
// The indexer query of every sequence: bf16 q[B][32][128] (q_scales null),
// or MXFP4 planes q[B][32][64] codes + q_scales[B][32][4]; weights w[B][32].
struct IndexQuery {
  const void* q;
  const uint8_t* q_scales;
  const float* w;
};
hipError_t launch_indexer(int keyfmt, const void* k_codes,
                          const uint8_t* k_scales, int64_t n_cap,
                          const int32_t* n_entries, const int32_t* cand,
                          int64_t n_rows, const IndexQuery& iq, int B,
                          float* scores, hipStream_t s,
                          uint32_t* tmax = nullptr, uint32_t* bmax = nullptr,
                          uint32_t* btmax = nullptr, int n_div = 1);

// The decode scan with local candidates (indexer_kernel LOCAL, MXFP4 keys):
// selection keys of every row into keys[B][round32(n_cap)], and per group
// of rows (a wavefront's tpw * 32 rows, or a workgroup's tpw * 128) its
// local top-kloc (key, id) pairs into lcand[B][n_wg][kloc] and a bound on
// what it left out into lbound[B][n_wg] (n_wg = groups per row).
// local_plan() picks the wavefront length, the group and kloc (2k pairs in
// all, at most kLocalMaxCands); ok is false when the row is too long.
// With candidate ids (cand [B][n_rows], as launch_indexer's) the rows are
// the candidates, the keys go to keys[B][round32(n_rows)] and the pairs
// carry the entry ids.  keyfmt 1 (bf16): the rows are bf16 block
// keys (k_codes; blocks of n_div entries, so ceil(n_entries / n_div) rows
// are valid), without candidate ids.
constexpr int kLocalMaxCands = 4096;
struct LocalPlan {
  bool ok = false;
  bool per_wave = false;
  int tpw = 8;
  int n_wg = 0;
  int kloc = 0;
};
LocalPlan local_plan(int B, int64_t n_cap, int k, bool qfp4,
                     bool cand = false, int max_cands = kLocalMaxCands);
hipError_t launch_indexer_local(const uint8_t* k_codes,
                                const uint8_t* k_scales, int64_t n_cap,
                                const int32_t* n_entries,
                                const IndexQuery& iq, int B, uint32_t* keys,
                                const LocalPlan& lp, uint2* lcand,
                                uint32_t* lbound, hipStream_t s,
                                const int32_t* cand = nullptr,
                                int64_t n_rows = 0,
                                int keyfmt = 0, int n_div = 1);

// topk.hip
// Exact per-row top-k (see topk.hip) of float scores (keys == false) or of
// selection keys (keys == true); rows of n_cols entries at stride ld (keys:
// ld a multiple of 32), ids (nullable) at stride n_cols; `tmax` (tile maxima
// [B][ceil(n_cols/32)] in the same form, nullable) enables tile pruning.
// A row's length is min(n_cols, ceil(n_valid[b] / valid_div)) when n_valid
// is given.
// With split_ws (split_workspace() bytes) and a row long enough to split
// (split_plan), the two-stage selection runs instead (see topk.hip).
hipError_t launch_row_select(const void* scores, const void* tmax, bool keys,
                             int64_t ld, int64_t n_cols, const int32_t* n_valid,
                             const int32_t* ids, int B, int k, int block,
                             const int32_t* limit, int32_t* out,
                             hipStream_t s, int valid_div = 1,
                             void* split_ws = nullptr);
struct SplitPlan {
  bool ok = false;
  int G = 0, kl = 0;          // chunks per row, pairs kept per chunk
};
SplitPlan split_plan(int B, int64_t n_cols, int k);
size_t split_workspace(int B, int64_t n_cols, int k);

// Two key selections (no ids) over the same B rows in one launch, side by
// side: rows of r0 on workgroups 0..B-1, rows of r1 on B..2B-1.
struct KeyRows {
  const void* keys;         // [B][ld] selection keys, ld a multiple of 32
  const void* tmax;         // [B][ceil(n_cols/32)] or null
  int64_t ld, n_cols;
  const int32_t* n_valid;   // nullable
  int k, block;
  const int32_t* limit;     // nullable
  int32_t* out;             // [B][k * block]
};
hipError_t launch_row_select_pair(const KeyRows& r0, const KeyRows& r1, int B,
                                  hipStream_t s);
// Standalone top-k over a score array (the two-stage selection, or tile
// maxima in `ws` for the one-workgroup-per-row selection).
size_t topk_workspace(int B, int64_t ld, int k);
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid,
                       const int32_t* ids, int B, int k, int block,
                       const int32_t* limit, int32_t* out, void* ws,
                       hipStream_t s);

// Benchmark hook of csa2_set_launch_events: the caller's events, recorded
// on the call's stream before its first kernel and after each kernel.
struct LaunchMarks {
  hipStream_t s;
  int i = 0;
  hipError_t mark();            // records the next event, if one is set
};

// attn.hip
int attn_splits(int B, int k);
size_t attn_workspace(int B, int k);
// Optional output details of the attention: a per-head sink logit in the
// softmax denominator, and the partial-RoPE de-rotation of the last 64
// output dims by the query position (pair i turns by -pos * rope_w[i]).
struct AttnEpilogue {
  const float* sink = nullptr;     // [64] logits, or null
  const int32_t* pos = nullptr;    // [B] query positions, or null
  double rope_w[32] = {};          // frequencies of the 32 pairs
};
// A fused selection: each attention workgroup first selects its sequence's
// top-k itself from the local candidates of launch_indexer_local (the exact
// block selection over the whole key row when the candidates cannot be
// shown to hold it), writes it to topk_out, then attends over it; `topk` is
// then unused.
struct FusedSelect {
  const uint2* lcand;          // [B][n_wg][kloc]
  const uint32_t* lbound;      // [B][n_wg]
  int n_wg, kloc;
  const uint32_t* keys;        // [B][ld] selection keys
  int64_t ld;
  const int32_t* n_entries;    // [B]
  int32_t* topk_out;           // [B][k]
  // Candidate rows (a pool): the keys row covers ids[B][n_ids] and the
  // fallback streams those rows with their entry ids (n_entries unused).
  const int32_t* ids = nullptr;
  int64_t n_ids = 0;
};
constexpr int kCandTopkMax = 8192;
// Exact top-k of the local candidates of launch_indexer_local (at most
// kCandTopkMax pairs per sequence; the fused selection's test and
// its exact fallback over keys[B][ld], whose first ceil(n_entries[b] /
// n_div) rows, at most n_rows, are visible), each chosen id expanded by
// `block` into out[B][k * block] (positions at or past limit[b] -> -1;
// ascending, -1 padded).  One workgroup per sequence.
hipError_t launch_cand_topk(const uint2* lcand, const uint32_t* lbound,
                            int n_wg, int kloc, const uint32_t* keys,
                            int64_t ld, int64_t n_rows,
                            const int32_t* n_entries, int n_div, int B, int k,
                            int block, const int32_t* limit, int32_t* out,
                            hipStream_t s);
hipError_t launch_attn(const uint8_t* main_codes, const uint8_t* main_scales,
                       int64_t n_cap, const int32_t* topk, int k,
                       const uint16_t* q, const uint8_t* swa,
                       const int32_t* n_swa, int B, float scale,
                       uint16_t* out, void* ws, hipStream_t s,
                       const AttnEpilogue& epi = AttnEpilogue{},
                       const FusedSelect* fsel = nullptr,
                       LaunchMarks* marks = nullptr);

// compress.hip
// Workspace bytes of launch_compress (slice partials of the projections).
size_t compress_workspace(int B, int m, int d);
// The decode-time write path for B sequences: hidden rows h[B][m][d] (bf16)
// -> C, Z (W^KV, W^Z: [512][d] bf16), C_bar (softmax pooling over the m
// tokens), K^I = C_bar W^IK ([128][512] bf16), packed into row rows[b] of
// each sequence's caches (skipped when outside [0, n_cap)), and the m rows
// C_i into window slots (swa_slot[b] + i) mod 128 when swa is set.
// cbar_out [B][512], ki_out [B][128], c_out [B][m][512] are optional.
hipError_t launch_compress(const uint16_t* h, int B, int m, int d,
                           const uint16_t* w_kv, const uint16_t* w_z,
                           const uint16_t* w_ik, const int32_t* rows,
                           int64_t n_cap, uint8_t* main_codes,
                           uint8_t* main_scales, uint8_t* idx_codes,
                           uint8_t* idx_scales, uint8_t* swa,
                           const int32_t* swa_slot, float* cbar_out,
                           float* ki_out, float* c_out, void* ws,
                           hipStream_t s);

}  // namespace csa2
