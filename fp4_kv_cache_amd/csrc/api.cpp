// libcsa2 C ABI: argument validation, workspace layout and the enqueue
// order of each call.  Every check happens before the first launch; on
// failure nothing is enqueued and a thread-local message is kept.
#include <cmath>
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "csa2.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

csa2_status fail(csa2_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

csa2_status hip_fail(hipError_t e, const char* what) {
  return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Records the next launch event (csa2_set_launch_events), if one is set.
#define CSA2_MARK(lm)                                                   \
  do {                                                                  \
    const hipError_t me_ = (lm).mark();                                 \
    if (me_ != hipSuccess) return hip_fail(me_, "launch event record"); \
  } while (0)


inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Device present and current?
csa2_status need_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "no HIP device");
  return CSA2_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  const uintptr_t y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr int kMaxK = 2048;
constexpr int kMaxBlock = 64;
constexpr int64_t kMaxCap = INT32_MAX;
// The indexer and attention address rows by 32-bit byte offsets within a
// sequence (up to 256 bytes per row).
constexpr int64_t kMaxAttnCap = int64_t(1) << 24;

// Workspace layout of csa2_sparse_attn_decode.
struct DecodeLayout {
  bool pool;
  int64_t nb = 0, n_cand = 0;
  int kb = 0;
  size_t off_scores = 0, off_tmax = 0, off_bscores = 0,
         off_pool = 0, off_pscores = 0, off_lcand = 0, off_lbound = 0,
         off_blcand = 0, off_blbound = 0, off_split = 0, off_attn = 0,
         total = 0;
};

inline size_t tiles_of(int64_t rows) { return (size_t)((rows + 31) / 32); }

// Key rows in the decode workspace are padded to a multiple of 32 entries.
int64_t round32(int64_t n) { return (n + 31) & ~(int64_t)31; }

DecodeLayout decode_layout(int B, int64_t n_cap, int k,
                           const csa2_pool_opts* pool) {
  DecodeLayout L;
  L.pool = pool != nullptr;
  size_t off = 0;
  if (!L.pool) {
    L.off_scores = off;
    off += align256((size_t)B * round32(n_cap) * 4);
    L.off_tmax = off;
    off += align256((size_t)B * tiles_of(n_cap) * 4);
    // Local candidates and bounds of the fused selection (at most
    // kLocalMaxCands pairs and kLocalMaxCands / 8 groups per sequence).
    L.off_lcand = off;
    off += align256((size_t)B * csa2::kLocalMaxCands * 8);
    L.off_lbound = off;
    off += align256((size_t)B * (csa2::kLocalMaxCands / 8) * 4);
    // The two-stage selection, for rows the fused selection cannot take.
    L.off_split = off;
    off += csa2::split_workspace(B, n_cap, k);
  } else {
    L.nb = (n_cap + pool->block - 1) / pool->block;
    L.kb = (int)std::min<int64_t>(pool->n_blocks_keep, L.nb);
    if (L.kb < 1) L.kb = 1;
    L.n_cand = (int64_t)L.kb * pool->block;
    L.off_bscores = off;
    off += align256((size_t)B * round32(L.nb) * 4);
    L.off_pool = off;
    off += align256((size_t)B * L.n_cand * 4);
    L.off_pscores = off;
    off += align256((size_t)B * round32(L.n_cand) * 4);
    L.off_tmax = off;
    off += align256((size_t)B * std::max(tiles_of(L.nb), tiles_of(L.n_cand)) * 4);
    // The two-stage selections of the blocks, then of the pool (one after
    // the other, so they share the space).
    L.off_split = off;
    off += std::max(csa2::split_workspace(B, L.nb, L.kb),
                    csa2::split_workspace(B, L.n_cand, k));
    // Local candidates of the pool scan for the fused selection.
    L.off_lcand = off;
    off += align256((size_t)B * csa2::kLocalMaxCands * 8);
    L.off_lbound = off;
    off += align256((size_t)B * (csa2::kLocalMaxCands / 8) * 4);
    // Local candidates of the block scan for the block selection.
    L.off_blcand = off;
    off += align256((size_t)B * csa2::kCandTopkMax * 8);
    L.off_blbound = off;
    off += align256((size_t)B * (csa2::kCandTopkMax / 8) * 4);
  }
  L.off_attn = off;
  off += align256(csa2::attn_workspace(B, k));
  L.total = off;
  return L;
}

// Workspace of csa2_full_pool_decode: keys, tile maxima, block maxima and
// their 32-block maxima, attention partials.
struct FullPoolLayout {
  int64_t nb = 0;
  size_t off_scores = 0, off_tmax = 0, off_bmax = 0, off_btmax = 0,
         off_split = 0, off_split_b = 0, off_attn = 0, total = 0;
};
FullPoolLayout full_pool_layout(int B, int64_t n_cap, int k, int kb) {
  FullPoolLayout L;
  L.nb = (n_cap + 7) / 8;
  size_t off = 0;
  L.off_scores = off;
  off += align256((size_t)B * round32(n_cap) * 4);
  L.off_tmax = off;
  off += align256((size_t)B * tiles_of(n_cap) * 4);
  L.off_bmax = off;
  off += align256((size_t)B * round32(L.nb) * 4);
  L.off_btmax = off;
  off += align256((size_t)B * tiles_of(L.nb) * 4);
  // The two-stage selections of the layer's top-k and of the blocks.
  L.off_split = off;
  off += csa2::split_workspace(B, n_cap, k);
  L.off_split_b = off;
  off += csa2::split_workspace(B, L.nb, kb);
  L.off_attn = off;
  off += align256(csa2::attn_workspace(B, k));
  L.total = off;
  return L;
}

// Workspace of csa2_reindex_decode: pool keys, their tile maxima, attention.
struct ReindexLayout {
  size_t off_scores = 0, off_tmax = 0, off_split = 0, off_lcand = 0,
         off_lbound = 0, off_attn = 0, total = 0;
};
ReindexLayout reindex_layout(int B, int64_t n_pool, int k) {
  ReindexLayout L;
  size_t off = 0;
  L.off_scores = off;
  off += align256((size_t)B * round32(n_pool) * 4);
  L.off_tmax = off;
  off += align256((size_t)B * tiles_of(n_pool) * 4);
  L.off_split = off;
  off += csa2::split_workspace(B, n_pool, k);
  L.off_lcand = off;
  off += align256((size_t)B * csa2::kLocalMaxCands * 8);
  L.off_lbound = off;
  off += align256((size_t)B * (csa2::kLocalMaxCands / 8) * 4);
  L.off_attn = off;
  off += align256(csa2::attn_workspace(B, k));
  L.total = off;
  return L;
}

constexpr int64_t kMaxPool = int64_t(1) << 26;

csa2_status check_pool(const csa2_pool_opts* pool) {
  if (!pool) return CSA2_OK;
  if (pool->n_blocks_keep < 1 || pool->block < 1 || pool->block > kMaxBlock)
    return fail(CSA2_ERR_UNSUPPORTED,
                "pool: n_blocks_keep must be >= 1 and block in 1..%d",
                kMaxBlock);
  if ((int64_t)pool->n_blocks_keep * pool->block > (int64_t)1 << 26)
    return fail(CSA2_ERR_UNSUPPORTED, "pool: n_blocks_keep * block too large");
  return CSA2_OK;
}

csa2_status check_attn_common(const uint8_t* main_codes,
                              const uint8_t* main_scales, int64_t n_cap,
                              const uint16_t* q, const uint8_t* swa,
                              const int32_t* n_swa, int32_t B, int32_t k,
                              float scale, const uint16_t* out) {
  if (B < 0) return fail(CSA2_ERR_INVALID_ARG, "B must be >= 0");
  if (k < 1 || k > kMaxK)
    return fail(CSA2_ERR_UNSUPPORTED, "k must be in 1..%d (got %d)", kMaxK, k);
  if (n_cap < 0 || n_cap > kMaxCap)
    return fail(CSA2_ERR_INVALID_ARG, "n_cap must be in 0..2^31-1");
  if (n_cap > kMaxAttnCap)
    return fail(CSA2_ERR_UNSUPPORTED,
                "attention needs n_cap <= 2^24 (got %lld)", (long long)n_cap);
  if (!std::isfinite(scale) || scale == 0.0f)
    return fail(CSA2_ERR_INVALID_ARG, "scale must be a finite nonzero float");
  if (B == 0) return CSA2_OK;
  if (!main_codes || !main_scales || !q || !swa || !n_swa || !out)
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(main_codes, 16) || !aligned(q, 16) || !aligned(out, 16) ||
      !aligned(swa, 16) || !aligned(main_scales, 4) || !aligned(n_swa, 4))
    return fail(CSA2_ERR_ALIGNMENT,
                "main_codes, q, out, swa need 16-byte and main_scales, "
                "n_swa 4-byte alignment");
  const size_t out_bytes = (size_t)B * 64 * 512 * 2;
  if (overlap(out, out_bytes, q, out_bytes) ||
      overlap(out, out_bytes, swa, (size_t)B * 128 * 512) ||
      overlap(out, out_bytes, main_codes, (size_t)B * n_cap * 256))
    return fail(CSA2_ERR_INVALID_ARG, "out overlaps an input");
  return CSA2_OK;
}

}  // namespace

extern "C" {

// csa2_set_launch_events: the caller's events for the next calls.
namespace {
constexpr int kMaxLaunchEvents = 16;
void* g_launch_events[kMaxLaunchEvents] = {};
int g_n_launch_events = 0;
int g_n_recorded = 0;           // events recorded by the latest call
}  // namespace

csa2_status csa2_set_launch_events(void* const* events, int32_t n) {
  if (n < 0 || n > kMaxLaunchEvents || (n > 0 && !events))
    return fail(CSA2_ERR_INVALID_ARG, "launch events: need 0 <= n <= %d and "
                "an array when n > 0", kMaxLaunchEvents);
  for (int i = 0; i < n; ++i) g_launch_events[i] = events[i];
  g_n_launch_events = n;
  return CSA2_OK;
}

int32_t csa2_launch_events_recorded(void) { return g_n_recorded; }

}  // extern "C"

hipError_t csa2::LaunchMarks::mark() {
  const int j = i++;
  if (j == 0) g_n_recorded = 0;
  if (j >= g_n_launch_events) return hipSuccess;
  g_n_recorded = j + 1;
  return hipEventRecord(static_cast<hipEvent_t>(g_launch_events[j]), s);
}

extern "C" {

const char* csa2_last_error(void) { return g_err; }

const char* csa2_version(void) { return "libcsa2 0.1.0 (gfx950)"; }

int32_t csa2_entry_bytes(int32_t fmt) {
  switch (fmt) {
    case CSA2_FMT_MAIN: return 256 + 32;
    case CSA2_FMT_IDX: return 64 + 4;
    case CSA2_FMT_SWA: return 512;
    default: return -1;
  }
}

double csa2_kv_bytes_per_token(const int32_t* m, int32_t n) {
  if (!m || n < 0) return -1.0;
  const double entry = csa2_entry_bytes(CSA2_FMT_MAIN) + csa2_entry_bytes(CSA2_FMT_IDX);
  double s = 0.0;
  for (int i = 0; i < n; ++i) {
    if (m[i] < 1) return -1.0;
    s += entry / m[i];
  }
  return s;
}

size_t csa2_workspace_size(int32_t op, int32_t B, int64_t n_cap, int32_t k,
                           const csa2_pool_opts* pool) {
  if (op == CSA2_OP_COMPRESS) {     // n_cap = m, k = d
    if (B < 0 || n_cap < 1 || n_cap > 16 || k < 16 || k > 16384 || k % 16)
      return 0;
    return csa2::compress_workspace(B, (int)n_cap, k);
  }
  if (B < 0 || n_cap < 0 || n_cap > kMaxCap || k < 1 || k > kMaxK) return 0;
  switch (op) {
    case CSA2_OP_TOPK:
      return csa2::topk_workspace(B, n_cap, k);
    case CSA2_OP_DECODE:
      if (pool && (pool->block < 1 || pool->block > kMaxBlock ||
                   pool->n_blocks_keep < 1))
        return 0;
      return decode_layout(B, n_cap, k, pool).total;
    case CSA2_OP_REUSE:
      return csa2::attn_workspace(B, k);
    case CSA2_OP_FULL_POOL:
      if (!pool || pool->block != 8 || pool->n_blocks_keep < 1 ||
          pool->n_blocks_keep > kMaxK)
        return 0;
      return full_pool_layout(B, n_cap, k, pool->n_blocks_keep).total;
    case CSA2_OP_REINDEX:
      if (n_cap < 1 || n_cap > kMaxPool) return 0;
      return reindex_layout(B, n_cap, k).total;
    case CSA2_OP_COMPRESS:
      return 0;     // handled above
    default:
      return 0;
  }
}

csa2_status csa2_pack_kv(int32_t fmt, const float* src, int64_t n_rows,
                         void* dst_codes, void* dst_scales, void* stream) {
  if (fmt != CSA2_FMT_MAIN && fmt != CSA2_FMT_IDX && fmt != CSA2_FMT_SWA)
    return fail(CSA2_ERR_INVALID_ARG, "unknown format %d", fmt);
  if (n_rows < 0) return fail(CSA2_ERR_INVALID_ARG, "n_rows must be >= 0");
  if (n_rows == 0) return CSA2_OK;
  if (!src || !dst_codes)
    return fail(CSA2_ERR_INVALID_ARG, "null src or dst_codes");
  if (fmt == CSA2_FMT_SWA && dst_scales)
    return fail(CSA2_ERR_INVALID_ARG, "CSA2_FMT_SWA has no scale plane");
  if (fmt != CSA2_FMT_SWA && !dst_scales)
    return fail(CSA2_ERR_INVALID_ARG, "null dst_scales");
  if (!aligned(src, 16) || !aligned(dst_codes, 16))
    return fail(CSA2_ERR_ALIGNMENT, "src and dst_codes need 16-byte alignment");
  const int dim = fmt == CSA2_FMT_IDX ? 128 : 512;
  const size_t cb = (size_t)n_rows * (fmt == CSA2_FMT_MAIN ? 256 : (fmt == CSA2_FMT_IDX ? 64 : 512));
  const size_t sb = (size_t)n_rows * (fmt == CSA2_FMT_MAIN ? 32 : 4);
  if (overlap(src, (size_t)n_rows * dim * 4, dst_codes, cb) ||
      (dst_scales && overlap(src, (size_t)n_rows * dim * 4, dst_scales, sb)) ||
      (dst_scales && overlap(dst_codes, cb, dst_scales, sb)))
    return fail(CSA2_ERR_INVALID_ARG, "buffers overlap");
  csa2_status st = need_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (fmt == CSA2_FMT_MAIN)
    e = csa2::launch_pack_main(src, n_rows, static_cast<uint8_t*>(dst_codes),
                               static_cast<uint8_t*>(dst_scales), s);
  else if (fmt == CSA2_FMT_IDX)
    e = csa2::launch_pack_idx(src, n_rows, static_cast<uint8_t*>(dst_codes),
                              static_cast<uint8_t*>(dst_scales), s);
  else
    e = csa2::launch_pack_swa(src, n_rows, static_cast<uint8_t*>(dst_codes), s);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "csa2_pack_kv launch");
}

csa2_status csa2_unpack_kv(int32_t fmt, const void* codes, const void* scales,
                           int64_t n_rows, float* dst, void* stream) {
  if (fmt != CSA2_FMT_MAIN && fmt != CSA2_FMT_IDX && fmt != CSA2_FMT_SWA)
    return fail(CSA2_ERR_INVALID_ARG, "unknown format %d", fmt);
  if (n_rows < 0) return fail(CSA2_ERR_INVALID_ARG, "n_rows must be >= 0");
  if (n_rows == 0) return CSA2_OK;
  if (!codes || !dst || (fmt != CSA2_FMT_SWA && !scales))
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(dst, 8)) return fail(CSA2_ERR_ALIGNMENT, "dst needs 8-byte alignment");
  csa2_status st = need_device();
  if (st) return st;
  hipError_t e = csa2::launch_unpack(fmt, static_cast<const uint8_t*>(codes),
                                     static_cast<const uint8_t*>(scales),
                                     n_rows, dst, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "csa2_unpack_kv launch");
}

csa2_status csa2_build_block_keys(const uint8_t* idx_codes,
                                  const uint8_t* idx_scales, int64_t n_cap,
                                  const int32_t* n_entries, int32_t B,
                                  int32_t block, uint16_t* block_keys,
                                  void* stream) {
  if (B < 0 || n_cap < 0 || n_cap > kMaxCap)
    return fail(CSA2_ERR_INVALID_ARG, "bad B or n_cap");
  if (block < 1 || block > kMaxBlock)
    return fail(CSA2_ERR_UNSUPPORTED, "block must be in 1..%d", kMaxBlock);
  if (B == 0 || n_cap == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !n_entries || !block_keys)
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  csa2_status st = need_device();
  if (st) return st;
  hipError_t e = csa2::launch_block_keys(idx_codes, idx_scales, n_cap,
                                         n_entries, B, block, block_keys,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "csa2_build_block_keys launch");
}

namespace {
// The attention epilogue of csa2_attn_opts: pair frequencies in double,
// rope_theta^(-2i/64).
csa2_status make_epilogue(const csa2_attn_opts* o, csa2::AttnEpilogue& epi) {
  epi = csa2::AttnEpilogue{};
  if (!o) return CSA2_OK;
  if (o->sink && !aligned(o->sink, 4))
    return fail(CSA2_ERR_ALIGNMENT, "sink needs 4-byte alignment");
  if (o->pos) {
    if (!aligned(o->pos, 4))
      return fail(CSA2_ERR_ALIGNMENT, "pos needs 4-byte alignment");
    if (!(o->rope_theta > 0.0f) || !std::isfinite(o->rope_theta))
      return fail(CSA2_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
    for (int i = 0; i < 32; ++i)
      epi.rope_w[i] = std::pow((double)o->rope_theta, -2.0 * i / 64.0);
  }
  epi.sink = o->sink;
  epi.pos = o->pos;
  return CSA2_OK;
}

// Checks the indexer query (bf16, or MXFP4 planes when q_scales is set).
csa2_status check_query(const csa2::IndexQuery& iq) {
  if (!iq.q || !iq.w) return fail(CSA2_ERR_INVALID_ARG, "null indexer query");
  if (!aligned(iq.q, 16) || !aligned(iq.w, 4) ||
      (iq.q_scales && !aligned(iq.q_scales, 4)))
    return fail(CSA2_ERR_ALIGNMENT, "the indexer query needs 16-byte "
                "(codes) and 4-byte (scales, w) alignment");
  return CSA2_OK;
}
size_t query_bytes(const csa2::IndexQuery& iq, int32_t B) {
  return (size_t)B * 32 * (iq.q_scales ? 64 : 256);
}

csa2_status indexer_score_impl(int32_t keyfmt, const void* k_codes,
                               const void* k_scales, int64_t n_cap,
                               const int32_t* n_entries, const int32_t* cand,
                               int32_t n_cand, const csa2::IndexQuery& iq,
                               int32_t B, float* scores, void* stream) {
  if (keyfmt != CSA2_KEYS_MXFP4 && keyfmt != CSA2_KEYS_BF16)
    return fail(CSA2_ERR_INVALID_ARG, "unknown key format %d", keyfmt);
  if (B < 0 || n_cap < 0 || n_cap > kMaxCap || (cand && n_cand < 0))
    return fail(CSA2_ERR_INVALID_ARG, "bad B, n_cap or n_cand");
  if (n_cap > kMaxAttnCap)
    return fail(CSA2_ERR_UNSUPPORTED,
                "the indexer needs n_cap <= 2^24 (got %lld)", (long long)n_cap);
  const int64_t rows = cand ? n_cand : n_cap;
  if (B == 0 || rows == 0) return CSA2_OK;
  if (!k_codes || !n_entries || !scores)
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  csa2_status qs = check_query(iq);
  if (qs) return qs;
  if (keyfmt == CSA2_KEYS_MXFP4 && !k_scales)
    return fail(CSA2_ERR_INVALID_ARG, "MXFP4 keys need k_scales");
  if (keyfmt == CSA2_KEYS_BF16 && k_scales)
    return fail(CSA2_ERR_INVALID_ARG, "bf16 keys take no k_scales");
  if (!aligned(k_codes, 16) || !aligned(scores, 4) ||
      (k_scales && !aligned(k_scales, 4)))
    return fail(CSA2_ERR_ALIGNMENT,
                "k_codes needs 16-byte, k_scales and scores 4-byte alignment");
  const size_t kbytes = (size_t)B * n_cap * (keyfmt == CSA2_KEYS_MXFP4 ? 64 : 256);
  if (overlap(scores, (size_t)B * rows * 4, k_codes, kbytes) ||
      overlap(scores, (size_t)B * rows * 4, iq.q, query_bytes(iq, B)))
    return fail(CSA2_ERR_INVALID_ARG, "scores overlap an input");
  csa2_status st = need_device();
  if (st) return st;
  hipError_t e = csa2::launch_indexer(
      keyfmt, k_codes, static_cast<const uint8_t*>(k_scales), n_cap, n_entries,
      cand, rows, iq, B, scores, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "csa2_indexer_score launch");
}
}  // namespace

csa2_status csa2_indexer_score(int32_t keyfmt, const void* k_codes,
                               const void* k_scales, int64_t n_cap,
                               const int32_t* n_entries, const int32_t* cand,
                               int32_t n_cand, const uint16_t* q_idx,
                               const float* w, int32_t B, float* scores,
                               void* stream) {
  return indexer_score_impl(keyfmt, k_codes, k_scales, n_cap, n_entries, cand,
                            n_cand, csa2::IndexQuery{q_idx, nullptr, w}, B,
                            scores, stream);
}

csa2_status csa2_indexer_score_fp4q(int32_t keyfmt, const void* k_codes,
                                    const void* k_scales, int64_t n_cap,
                                    const int32_t* n_entries,
                                    const int32_t* cand, int32_t n_cand,
                                    const uint8_t* q_codes,
                                    const uint8_t* q_scales, const float* w,
                                    int32_t B, float* scores, void* stream) {
  if (!q_scales && q_codes)
    return fail(CSA2_ERR_INVALID_ARG, "an MXFP4 query needs q_scales");
  return indexer_score_impl(keyfmt, k_codes, k_scales, n_cap, n_entries, cand,
                            n_cand, csa2::IndexQuery{q_codes, q_scales, w}, B,
                            scores, stream);
}

csa2_status csa2_topk(const float* scores, int64_t ld, const int32_t* n_valid,
                      const int32_t* ids, int32_t B, int32_t k, int32_t block,
                      const int32_t* limit, int32_t* out, void* ws,
                      size_t ws_bytes, void* stream) {
  if (B < 0 || ld < 1 || ld > kMaxCap)
    return fail(CSA2_ERR_INVALID_ARG, "bad B or ld");
  if (k < 1 || k > kMaxK)
    return fail(CSA2_ERR_UNSUPPORTED, "k must be in 1..%d (got %d)", kMaxK, k);
  if (block < 1 || block > kMaxBlock)
    return fail(CSA2_ERR_UNSUPPORTED, "block must be in 1..%d", kMaxBlock);
  if (B == 0) return CSA2_OK;
  if (!scores || !out) return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(scores, 4) || !aligned(out, 4))
    return fail(CSA2_ERR_ALIGNMENT, "scores and out need 4-byte alignment");
  const size_t need = csa2::topk_workspace(B, ld, k);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(CSA2_ERR_WORKSPACE, "topk needs %zu bytes of 256-byte aligned "
                "workspace (got %zu)", need, ws_bytes);
  if (overlap(out, (size_t)B * k * block * 4, scores, (size_t)B * ld * 4))
    return fail(CSA2_ERR_INVALID_ARG, "out overlaps scores");
  csa2_status st = need_device();
  if (st) return st;
  hipError_t e = csa2::launch_topk(scores, ld, n_valid, ids, B, k, block,
                                   limit, out, ws,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "csa2_topk launch");
}

csa2_status csa2_reuse_attn(const uint8_t* main_codes,
                            const uint8_t* main_scales, int64_t n_cap,
                            const int32_t* topk, int32_t k, const uint16_t* q,
                            const uint8_t* swa, const int32_t* n_swa,
                            int32_t B, float scale, uint16_t* out, void* ws,
                            size_t ws_bytes, void* stream) {
  return csa2_reuse_attn_ex(main_codes, main_scales, n_cap, topk, k, q, swa,
                            n_swa, B, scale, nullptr, out, ws, ws_bytes,
                            stream);
}

csa2_status csa2_reuse_attn_ex(const uint8_t* main_codes,
                               const uint8_t* main_scales, int64_t n_cap,
                               const int32_t* topk, int32_t k,
                               const uint16_t* q, const uint8_t* swa,
                               const int32_t* n_swa, int32_t B, float scale,
                               const csa2_attn_opts* opts, uint16_t* out,
                               void* ws, size_t ws_bytes, void* stream) {
  csa2::AttnEpilogue epi;
  csa2_status est = make_epilogue(opts, epi);
  if (est) return est;
  csa2_status st = check_attn_common(main_codes, main_scales, n_cap, q, swa,
                                     n_swa, B, k, scale, out);
  if (st) return st;
  if (B == 0) return CSA2_OK;
  if (!topk) return fail(CSA2_ERR_INVALID_ARG, "null topk");
  const size_t need = csa2::attn_workspace(B, k);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(CSA2_ERR_WORKSPACE, "reuse needs %zu bytes of 256-byte aligned "
                "workspace (got %zu)", need, ws_bytes);
  st = need_device();
  if (st) return st;
  csa2::LaunchMarks lm{static_cast<hipStream_t>(stream)};
  CSA2_MARK(lm);
  hipError_t e = csa2::launch_attn(main_codes, main_scales, n_cap, topk, k, q,
                                   swa, n_swa, B, scale, out, ws,
                                   static_cast<hipStream_t>(stream), epi,
                                   nullptr, &lm);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "csa2_reuse_attn launch");
}

namespace {
csa2_status decode_impl(const csa2_cache* kv, const csa2::IndexQuery& iq,
                        const uint16_t* q, const uint8_t* swa,
                        const int32_t* n_swa, int32_t B, int32_t k,
                        float scale, const csa2_pool_opts* pool,
                        uint16_t* out, int32_t* topk_out, void* ws,
                        size_t ws_bytes, void* stream,
                        const csa2_attn_opts* opts = nullptr) {
  csa2::AttnEpilogue epi;
  csa2_status est = make_epilogue(opts, epi);
  if (est) return est;
  if (!kv) return fail(CSA2_ERR_INVALID_ARG, "null cache descriptor");
  csa2_status st = check_attn_common(kv->main_codes, kv->main_scales,
                                     kv->n_cap, q, swa, n_swa, B, k, scale, out);
  if (st) return st;
  st = check_pool(pool);
  if (st) return st;
  if (B == 0) return CSA2_OK;
  if (kv->n_cap < 1) return fail(CSA2_ERR_INVALID_ARG, "n_cap must be >= 1");
  if (!kv->idx_codes || !kv->idx_scales || !kv->n_entries || !topk_out)
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  st = check_query(iq);
  if (st) return st;
  if (pool && !kv->block_keys)
    return fail(CSA2_ERR_INVALID_ARG, "a pool needs kv->block_keys");
  if (!aligned(kv->idx_codes, 16) || !aligned(kv->idx_scales, 4) ||
      !aligned(topk_out, 4) ||
      (pool && !aligned(kv->block_keys, 16)))
    return fail(CSA2_ERR_ALIGNMENT, "misaligned indexer argument");
  const DecodeLayout L = decode_layout(B, kv->n_cap, k, pool);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(CSA2_ERR_WORKSPACE, "decode needs %zu bytes of 256-byte "
                "aligned workspace (got %zu)", L.total, ws_bytes);
  st = need_device();
  if (st) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  hipError_t e;
  csa2::LaunchMarks lm{s};
  CSA2_MARK(lm);
  // Decode-internal buffers hold selection keys (uint32), not scores.
  uint32_t* tmax = reinterpret_cast<uint32_t*>(base + L.off_tmax);
  const csa2::LocalPlan lp =
      pool ? csa2::LocalPlan{}
           : csa2::local_plan(B, kv->n_cap, k, iq.q_scales != nullptr);
  if (!pool && lp.ok) {
    // Scan with per-workgroup local candidates; the selection happens in
    // the attention workgroups themselves.
    uint32_t* keys = reinterpret_cast<uint32_t*>(base + L.off_scores);
    uint2* lcand = reinterpret_cast<uint2*>(base + L.off_lcand);
    uint32_t* lbound = reinterpret_cast<uint32_t*>(base + L.off_lbound);
    e = csa2::launch_indexer_local(kv->idx_codes, kv->idx_scales, kv->n_cap,
                                   kv->n_entries, iq, B, keys, lp, lcand,
                                   lbound, s);
    if (e != hipSuccess) return hip_fail(e, "indexer launch");
    CSA2_MARK(lm);
    const csa2::FusedSelect fs{lcand, lbound, lp.n_wg, lp.kloc, keys,
                               round32(kv->n_cap), kv->n_entries, topk_out};
    e = csa2::launch_attn(kv->main_codes, kv->main_scales, kv->n_cap,
                          topk_out, k, q, swa, n_swa, B, scale, out,
                          base + L.off_attn, s, epi, &fs, &lm);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return CSA2_OK;
  }
  if (!pool) {
    float* scores = reinterpret_cast<float*>(base + L.off_scores);
    e = csa2::launch_indexer(CSA2_KEYS_MXFP4, kv->idx_codes, kv->idx_scales,
                             kv->n_cap, kv->n_entries, nullptr, kv->n_cap,
                             iq, B, scores, s, tmax);
    if (e != hipSuccess) return hip_fail(e, "indexer launch");
    CSA2_MARK(lm);
    e = csa2::launch_row_select(scores, tmax, true, round32(kv->n_cap),
                                kv->n_cap, kv->n_entries, nullptr, B, k, 1,
                                nullptr, topk_out, s, 1, base + L.off_split);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    CSA2_MARK(lm);
  } else {
    float* bscores = reinterpret_cast<float*>(base + L.off_bscores);
    int32_t* pool_ids = reinterpret_cast<int32_t*>(base + L.off_pool);
    float* pscores = reinterpret_cast<float*>(base + L.off_pscores);
    // Blocks of `block` entries: sequence b has ceil(n_entries[b] / block)
    // of them, which the scan and the select work out themselves.
    const csa2::LocalPlan bp =
        csa2::local_plan(B, L.nb, L.kb, iq.q_scales != nullptr, false,
                         csa2::kCandTopkMax);
    if (bp.ok && bp.tpw == 8) {
      // The block scan keeps local candidates; one workgroup per sequence
      // then selects the blocks from them and expands the pool.
      uint32_t* bkeys = reinterpret_cast<uint32_t*>(bscores);
      uint2* blcand = reinterpret_cast<uint2*>(base + L.off_blcand);
      uint32_t* blbound = reinterpret_cast<uint32_t*>(base + L.off_blbound);
      e = csa2::launch_indexer_local(
          reinterpret_cast<const uint8_t*>(kv->block_keys), nullptr, L.nb,
          kv->n_entries, iq, B, bkeys, bp, blcand, blbound, s, nullptr, 0,
          CSA2_KEYS_BF16, pool->block);
      if (e != hipSuccess) return hip_fail(e, "block indexer launch");
      CSA2_MARK(lm);
      e = csa2::launch_cand_topk(blcand, blbound, bp.n_wg, bp.kloc, bkeys,
                                 round32(L.nb), L.nb, kv->n_entries,
                                 pool->block, B, L.kb, pool->block,
                                 kv->n_entries, pool_ids, s);
      if (e != hipSuccess) return hip_fail(e, "block top-k launch");
      CSA2_MARK(lm);
    } else {
      e = csa2::launch_indexer(CSA2_KEYS_BF16, kv->block_keys, nullptr, L.nb,
                               kv->n_entries, nullptr, L.nb, iq, B, bscores,
                               s, tmax, nullptr, nullptr, pool->block);
      if (e != hipSuccess) return hip_fail(e, "block indexer launch");
      CSA2_MARK(lm);
      e = csa2::launch_row_select(bscores, tmax, true, round32(L.nb), L.nb,
                                  kv->n_entries, nullptr, B, L.kb,
                                  pool->block, kv->n_entries, pool_ids, s,
                                  pool->block, base + L.off_split);
      if (e != hipSuccess) return hip_fail(e, "block top-k launch");
      CSA2_MARK(lm);
    }
    const csa2::LocalPlan pp = csa2::local_plan(B, L.n_cand, k,
                                                iq.q_scales != nullptr, true);
    if (pp.ok) {
      // The pool scan keeps local candidates; the attention workgroups
      // select the pool's top-k themselves.
      uint32_t* pkeys = reinterpret_cast<uint32_t*>(pscores);
      uint2* lcand = reinterpret_cast<uint2*>(base + L.off_lcand);
      uint32_t* lbound = reinterpret_cast<uint32_t*>(base + L.off_lbound);
      e = csa2::launch_indexer_local(kv->idx_codes, kv->idx_scales, kv->n_cap,
                                     kv->n_entries, iq, B, pkeys, pp, lcand,
                                     lbound, s, pool_ids, L.n_cand);
      if (e != hipSuccess) return hip_fail(e, "pool indexer launch");
      CSA2_MARK(lm);
      csa2::FusedSelect fs{lcand, lbound, pp.n_wg, pp.kloc, pkeys,
                           round32(L.n_cand), nullptr, topk_out};
      fs.ids = pool_ids;
      fs.n_ids = L.n_cand;
      e = csa2::launch_attn(kv->main_codes, kv->main_scales, kv->n_cap,
                            topk_out, k, q, swa, n_swa, B, scale, out,
                            base + L.off_attn, s, epi, &fs, &lm);
      if (e != hipSuccess) return hip_fail(e, "attention launch");
      return CSA2_OK;
    }
    e = csa2::launch_indexer(CSA2_KEYS_MXFP4, kv->idx_codes, kv->idx_scales,
                             kv->n_cap, kv->n_entries, pool_ids, L.n_cand,
                             iq, B, pscores, s, tmax);
    if (e != hipSuccess) return hip_fail(e, "pool indexer launch");
    CSA2_MARK(lm);
    e = csa2::launch_row_select(pscores, tmax, true, round32(L.n_cand),
                                L.n_cand, nullptr, pool_ids, B, k, 1, nullptr,
                                topk_out, s, 1, base + L.off_split);
    if (e != hipSuccess) return hip_fail(e, "pool top-k launch");
    CSA2_MARK(lm);
  }
  e = csa2::launch_attn(kv->main_codes, kv->main_scales, kv->n_cap, topk_out,
                        k, q, swa, n_swa, B, scale, out, base + L.off_attn, s,
                        epi, nullptr, &lm);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return CSA2_OK;
}
}  // namespace

csa2_status csa2_sparse_attn_decode(const csa2_cache* kv,
                                    const uint16_t* q_idx, const float* w,
                                    const uint16_t* q, const uint8_t* swa,
                                    const int32_t* n_swa, int32_t B, int32_t k,
                                    float scale, const csa2_pool_opts* pool,
                                    uint16_t* out, int32_t* topk_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  return decode_impl(kv, csa2::IndexQuery{q_idx, nullptr, w}, q, swa, n_swa,
                     B, k, scale, pool, out, topk_out, ws, ws_bytes, stream);
}

}  // extern "C"

// The decode workspace of csa2_sparse_attn_decode_noalloc: a fixed device
// array of the library, one copy per GPU, living until the process ends.
// Host code never passes `scratch` itself to a kernel (in host code the
// name is only a stand-in for the symbol): the device address of each GPU's
// copy is looked up once per device, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on first use).
csa2_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "no HIP device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CSA2_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "scratch symbol address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CSA2_OK;
}
}  // namespace

extern "C" {

csa2_status csa2_sparse_attn_decode_noalloc(
    const csa2_cache* kv, const uint16_t* q_idx, const float* w,
    const uint16_t* q, const uint8_t* swa, const int32_t* n_swa, int32_t B,
    int32_t k, float scale, const csa2_pool_opts* pool, uint16_t* out,
    int32_t* topk_out, void* stream) {
  if (B < 0 || !kv || kv->n_cap < 0 || kv->n_cap > kMaxCap || k < 1 ||
      k > kMaxK)
    return decode_impl(kv, csa2::IndexQuery{q_idx, nullptr, w}, q, swa,
                       n_swa, B, k, scale, pool, out, topk_out, nullptr, 0,
                       stream);                 // reports the argument error
  if (pool && check_pool(pool)) return CSA2_ERR_UNSUPPORTED;
  // Far beyond the scratch array anyway; keeps the layout sums in range.
  if ((uint64_t)B * (uint64_t)round32(kv->n_cap) > ((uint64_t)1 << 40))
    return fail(CSA2_ERR_WORKSPACE, "csa2_sparse_attn_decode_noalloc: B * "
                "n_cap is far beyond the %zu-byte scratch array",
                (size_t)CSA2_NOALLOC_SCRATCH_BYTES);
  const size_t need = decode_layout(B, kv->n_cap, k, pool).total;
  if (need > CSA2_NOALLOC_SCRATCH_BYTES)
    return fail(CSA2_ERR_WORKSPACE,
                "csa2_sparse_attn_decode_noalloc: this call needs %zu bytes "
                "of scratch, the library holds %zu (use "
                "csa2_sparse_attn_decode with a workspace)", need,
                (size_t)CSA2_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  csa2_status st = scratch_for_current_device(&ws);
  if (st) return st;
  // Nothing in the decode workspace has to start at zero: every kernel
  // writes what it later reads in the same call.
  return decode_impl(kv, csa2::IndexQuery{q_idx, nullptr, w}, q, swa, n_swa,
                     B, k, scale, pool, out, topk_out, ws,
                     CSA2_NOALLOC_SCRATCH_BYTES, stream);
}

csa2_status csa2_sparse_attn_decode_fp4q(
    const csa2_cache* kv, const uint8_t* q_codes, const uint8_t* q_scales,
    const float* w, const uint16_t* q, const uint8_t* swa,
    const int32_t* n_swa, int32_t B, int32_t k, float scale,
    const csa2_pool_opts* pool, uint16_t* out, int32_t* topk_out, void* ws,
    size_t ws_bytes, void* stream) {
  if (!q_scales && q_codes)
    return fail(CSA2_ERR_INVALID_ARG, "an MXFP4 query needs q_scales");
  return decode_impl(kv, csa2::IndexQuery{q_codes, q_scales, w}, q, swa,
                     n_swa, B, k, scale, pool, out, topk_out, ws, ws_bytes,
                     stream);
}

csa2_status csa2_sparse_attn_decode_fp4q_ex(
    const csa2_cache* kv, const uint8_t* q_codes, const uint8_t* q_scales,
    const float* w, const uint16_t* q, const uint8_t* swa,
    const int32_t* n_swa, int32_t B, int32_t k, float scale,
    const csa2_pool_opts* pool, const csa2_attn_opts* opts, uint16_t* out,
    int32_t* topk_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q_scales && q_codes)
    return fail(CSA2_ERR_INVALID_ARG, "an MXFP4 query needs q_scales");
  return decode_impl(kv, csa2::IndexQuery{q_codes, q_scales, w}, q, swa,
                     n_swa, B, k, scale, pool, out, topk_out, ws, ws_bytes,
                     stream, opts);
}

}  // extern "C"

csa2_status csa2_full_pool_decode(const csa2_cache* kv, const uint16_t* q_idx,
                                  const float* w, const uint16_t* q,
                                  const uint8_t* swa, const int32_t* n_swa,
                                  int32_t B, int32_t k, float scale,
                                  const csa2_pool_opts* pool, uint16_t* out,
                                  int32_t* topk_out, int32_t* pool_out,
                                  void* ws, size_t ws_bytes, void* stream) {
  return csa2_full_pool_decode_ex(kv, q_idx, w, q, swa, n_swa, B, k, scale,
                                  pool, nullptr, out, topk_out, pool_out, ws,
                                  ws_bytes, stream);
}

csa2_status csa2_full_pool_decode_ex(
    const csa2_cache* kv, const uint16_t* q_idx, const float* w,
    const uint16_t* q, const uint8_t* swa, const int32_t* n_swa, int32_t B,
    int32_t k, float scale, const csa2_pool_opts* pool,
    const csa2_attn_opts* opts, uint16_t* out, int32_t* topk_out,
    int32_t* pool_out, void* ws, size_t ws_bytes, void* stream) {
  csa2::AttnEpilogue epi;
  csa2_status est = make_epilogue(opts, epi);
  if (est) return est;
  if (!kv) return fail(CSA2_ERR_INVALID_ARG, "null cache descriptor");
  csa2_status st = check_attn_common(kv->main_codes, kv->main_scales,
                                     kv->n_cap, q, swa, n_swa, B, k, scale, out);
  if (st) return st;
  if (!pool) return fail(CSA2_ERR_INVALID_ARG, "null pool options");
  if (pool->block != 8 || pool->n_blocks_keep < 1 ||
      pool->n_blocks_keep > kMaxK)
    return fail(CSA2_ERR_UNSUPPORTED, "the pool needs block == 8 and "
                "n_blocks_keep in 1..%d", kMaxK);
  if (B == 0) return CSA2_OK;
  if (kv->n_cap < 1) return fail(CSA2_ERR_INVALID_ARG, "n_cap must be >= 1");
  if (!kv->idx_codes || !kv->idx_scales || !kv->n_entries || !topk_out ||
      !pool_out)
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  st = check_query(csa2::IndexQuery{q_idx, nullptr, w});
  if (st) return st;
  if (!aligned(kv->idx_codes, 16) || !aligned(kv->idx_scales, 4) ||
      !aligned(topk_out, 4) || !aligned(pool_out, 4))
    return fail(CSA2_ERR_ALIGNMENT, "misaligned indexer argument");
  const int64_t n_pool = (int64_t)pool->n_blocks_keep * 8;
  if (overlap(pool_out, (size_t)B * n_pool * 4, topk_out, (size_t)B * k * 4))
    return fail(CSA2_ERR_INVALID_ARG, "pool_out overlaps topk_out");
  const FullPoolLayout L =
      full_pool_layout(B, kv->n_cap, k, pool->n_blocks_keep);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(CSA2_ERR_WORKSPACE, "full-pool decode needs %zu bytes of "
                "256-byte aligned workspace (got %zu)", L.total, ws_bytes);
  st = need_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* scores = reinterpret_cast<float*>(base + L.off_scores);
  uint32_t* tmax = reinterpret_cast<uint32_t*>(base + L.off_tmax);
  uint32_t* bmax = reinterpret_cast<uint32_t*>(base + L.off_bmax);
  uint32_t* btmax = reinterpret_cast<uint32_t*>(base + L.off_btmax);
  hipError_t e = csa2::launch_indexer(
      CSA2_KEYS_MXFP4, kv->idx_codes, kv->idx_scales, kv->n_cap,
      kv->n_entries, nullptr, kv->n_cap, csa2::IndexQuery{q_idx, nullptr, w},
      B, scores, s, tmax, bmax, btmax);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  // The layer's own top-k, and beside it (same launch) the pool: the
  // n_blocks_keep blocks with the largest maximum, expanded to their
  // positions below n_entries (blocks past the end hold key 0 and are never
  // chosen).
  const csa2::KeyRows own{scores, tmax, round32(kv->n_cap), kv->n_cap,
                          kv->n_entries, k, 1, nullptr, topk_out};
  const csa2::KeyRows blocks{bmax, btmax, round32(L.nb), L.nb, nullptr,
                             pool->n_blocks_keep, 8, kv->n_entries, pool_out};
  if (csa2::split_plan(B, kv->n_cap, k).ok &&
      csa2::split_plan(B, L.nb, pool->n_blocks_keep).ok) {
    // Rows long enough for the two-stage selection: one after the other.
    e = csa2::launch_row_select(scores, nullptr, true, own.ld, own.n_cols,
                                own.n_valid, nullptr, B, own.k, own.block,
                                own.limit, own.out, s, 1, base + L.off_split);
    if (e == hipSuccess)
      e = csa2::launch_row_select(bmax, nullptr, true, blocks.ld,
                                  blocks.n_cols, blocks.n_valid, nullptr, B,
                                  blocks.k, blocks.block, blocks.limit,
                                  blocks.out, s, 1, base + L.off_split_b);
  } else {
    e = csa2::launch_row_select_pair(own, blocks, B, s);
  }
  if (e != hipSuccess) return hip_fail(e, "top-k and pool launch");
  e = csa2::launch_attn(kv->main_codes, kv->main_scales, kv->n_cap, topk_out,
                        k, q, swa, n_swa, B, scale, out, base + L.off_attn, s,
                        epi);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return CSA2_OK;
}

csa2_status csa2_reindex_decode(const csa2_cache* kv, const int32_t* pool,
                                int64_t n_pool, const uint16_t* q_idx,
                                const float* w, const uint16_t* q,
                                const uint8_t* swa, const int32_t* n_swa,
                                int32_t B, int32_t k, float scale,
                                uint16_t* out, int32_t* topk_out, void* ws,
                                size_t ws_bytes, void* stream) {
  return csa2_reindex_decode_ex(kv, pool, n_pool, q_idx, w, q, swa, n_swa, B,
                                k, scale, nullptr, out, topk_out, ws,
                                ws_bytes, stream);
}

csa2_status csa2_reindex_decode_ex(
    const csa2_cache* kv, const int32_t* pool, int64_t n_pool,
    const uint16_t* q_idx, const float* w, const uint16_t* q,
    const uint8_t* swa, const int32_t* n_swa, int32_t B, int32_t k,
    float scale, const csa2_attn_opts* opts, uint16_t* out,
    int32_t* topk_out, void* ws, size_t ws_bytes, void* stream) {
  csa2::AttnEpilogue epi;
  csa2_status est = make_epilogue(opts, epi);
  if (est) return est;
  if (!kv) return fail(CSA2_ERR_INVALID_ARG, "null cache descriptor");
  csa2_status st = check_attn_common(kv->main_codes, kv->main_scales,
                                     kv->n_cap, q, swa, n_swa, B, k, scale, out);
  if (st) return st;
  if (n_pool < 1 || n_pool > kMaxPool)
    return fail(CSA2_ERR_INVALID_ARG, "n_pool must be in 1..2^26");
  if (B == 0) return CSA2_OK;
  if (!kv->idx_codes || !kv->idx_scales || !kv->n_entries || !pool ||
      !topk_out)
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  st = check_query(csa2::IndexQuery{q_idx, nullptr, w});
  if (st) return st;
  if (!aligned(kv->idx_codes, 16) || !aligned(kv->idx_scales, 4) ||
      !aligned(pool, 4) || !aligned(topk_out, 4))
    return fail(CSA2_ERR_ALIGNMENT, "misaligned indexer argument");
  if (overlap(topk_out, (size_t)B * k * 4, pool, (size_t)B * n_pool * 4))
    return fail(CSA2_ERR_INVALID_ARG, "topk_out overlaps pool");
  const ReindexLayout L = reindex_layout(B, n_pool, k);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(CSA2_ERR_WORKSPACE, "reindex decode needs %zu bytes of "
                "256-byte aligned workspace (got %zu)", L.total, ws_bytes);
  st = need_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* scores = reinterpret_cast<float*>(base + L.off_scores);
  uint32_t* tmax = reinterpret_cast<uint32_t*>(base + L.off_tmax);
  const csa2::IndexQuery iq{q_idx, nullptr, w};
  hipError_t e;
  const csa2::LocalPlan pp = csa2::local_plan(B, n_pool, k, false, true);
  if (pp.ok) {
    // Local candidates of the pool, selected inside the attention.
    uint32_t* keys = reinterpret_cast<uint32_t*>(scores);
    uint2* lcand = reinterpret_cast<uint2*>(base + L.off_lcand);
    uint32_t* lbound = reinterpret_cast<uint32_t*>(base + L.off_lbound);
    e = csa2::launch_indexer_local(kv->idx_codes, kv->idx_scales, kv->n_cap,
                                   kv->n_entries, iq, B, keys, pp, lcand,
                                   lbound, s, pool, n_pool);
    if (e != hipSuccess) return hip_fail(e, "pool indexer launch");
    csa2::FusedSelect fs{lcand, lbound, pp.n_wg, pp.kloc, keys,
                         round32(n_pool), nullptr, topk_out};
    fs.ids = pool;
    fs.n_ids = n_pool;
    e = csa2::launch_attn(kv->main_codes, kv->main_scales, kv->n_cap,
                          topk_out, k, q, swa, n_swa, B, scale, out,
                          base + L.off_attn, s, epi, &fs);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return CSA2_OK;
  }
  e = csa2::launch_indexer(CSA2_KEYS_MXFP4, kv->idx_codes, kv->idx_scales,
                           kv->n_cap, kv->n_entries, pool, n_pool, iq, B,
                           scores, s, tmax);
  if (e != hipSuccess) return hip_fail(e, "pool indexer launch");
  e = csa2::launch_row_select(scores, tmax, true, round32(n_pool), n_pool,
                              nullptr, pool, B, k, 1, nullptr, topk_out, s, 1,
                              base + L.off_split);
  if (e != hipSuccess) return hip_fail(e, "pool top-k launch");
  e = csa2::launch_attn(kv->main_codes, kv->main_scales, kv->n_cap, topk_out,
                        k, q, swa, n_swa, B, scale, out, base + L.off_attn, s,
                        epi);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return CSA2_OK;
}

csa2_status csa2_sparse_attn_decode_ex(const csa2_cache* kv,
                                       const uint16_t* q_idx, const float* w,
                                       const uint16_t* q, const uint8_t* swa,
                                       const int32_t* n_swa, int32_t B,
                                       int32_t k, float scale,
                                       const csa2_pool_opts* pool,
                                       const csa2_attn_opts* opts,
                                       uint16_t* out, int32_t* topk_out,
                                       void* ws, size_t ws_bytes,
                                       void* stream) {
  return decode_impl(kv, csa2::IndexQuery{q_idx, nullptr, w}, q, swa, n_swa,
                     B, k, scale, pool, out, topk_out, ws, ws_bytes, stream,
                     opts);
}

csa2_status csa2_compress_append(const uint16_t* h, int32_t B, int32_t m,
                                 int32_t d, const uint16_t* w_kv,
                                 const uint16_t* w_z, const uint16_t* w_ik,
                                 const int32_t* rows, uint8_t* main_codes,
                                 uint8_t* main_scales, uint8_t* idx_codes,
                                 uint8_t* idx_scales, int64_t n_cap,
                                 uint8_t* swa, const int32_t* swa_slot,
                                 float* cbar_out, float* ki_out, float* c_out,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || n_cap < 1 || n_cap > kMaxCap)
    return fail(CSA2_ERR_INVALID_ARG, "bad B or n_cap");
  if (m < 1 || m > 16 || d < 16 || d > 16384 || d % 16)
    return fail(CSA2_ERR_UNSUPPORTED, "m must be in 1..16 and d a multiple "
                "of 16 in 16..16384");
  if (B == 0) return CSA2_OK;
  if (!h || !w_kv || !w_z || !w_ik || !rows || !main_codes || !main_scales ||
      !idx_codes || !idx_scales)
    return fail(CSA2_ERR_INVALID_ARG, "null pointer argument");
  if ((swa == nullptr) != (swa_slot == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "swa and swa_slot go together");
  if (!aligned(h, 16) || !aligned(w_kv, 16) || !aligned(w_z, 16) ||
      !aligned(w_ik, 16) || !aligned(rows, 4) || !aligned(main_codes, 16) ||
      !aligned(idx_codes, 16) || (swa_slot && !aligned(swa_slot, 4)) ||
      (cbar_out && !aligned(cbar_out, 4)) || (ki_out && !aligned(ki_out, 4)) ||
      (c_out && !aligned(c_out, 4)))
    return fail(CSA2_ERR_ALIGNMENT, "misaligned argument");
  const size_t need = csa2::compress_workspace(B, m, d);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(CSA2_ERR_WORKSPACE, "compress needs %zu bytes of 256-byte "
                "aligned workspace (got %zu)", need, ws_bytes);
  csa2_status st = need_device();
  if (st) return st;
  hipError_t e = csa2::launch_compress(
      h, B, m, d, w_kv, w_z, w_ik, rows, n_cap, main_codes, main_scales,
      idx_codes, idx_scales, swa, swa_slot, cbar_out, ki_out, c_out, ws,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "csa2_compress_append launch");
}
