/*
 * libcsa2 -- decode-time Compressed Sparse Attention 2 (CSA2) with an FP4
 * main-KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title; section / equation / table on them):
 *   [KVC]  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
 *          (mer.run post): 1 (setup list), 2 (entry sizes, B_global),
 *          4.1 (single-layer formulas), 4.2 (mode table), 4.3 (hierarchical
 *          indexer equation), 5 (FP4 quantiser equation).
 *   [ARCH] "DeepSeek-V4.1-Flash, 2. Architecture" course notes
 *          (guaifinition.github.io): 2.3 (CSA2), 2.3.1 (Full / Reindex /
 *          Reuse, Figure 4), 2.3.2 (hierarchical sparse indexer, Figure 5),
 *          2.4.4 (FP4 main KV cache).
 *   [V4]   "DeepSeek-V4: Towards Highly Efficient Million-Token Context
 *          Intelligence" (baisen.site): CSA step 2 (index score, top-k
 *          equations), CSA step 3 (shared-KV MQA equation), sliding window.
 *
 * Conventions for every call:
 *   - Buffer pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory; scratch comes from a caller
 *     workspace sized by csa2_workspace_size().
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls validate
 *     their arguments on the host, enqueue kernels and return without
 *     synchronising; results are ready when the stream is.
 *   - Per-sequence lengths (n_entries, n_swa, n_valid, limit) live in device
 *     memory and are read by the kernels; they must not exceed the host-side
 *     capacities passed alongside them.
 *   - Errors: every call returns a csa2_status.  Validation happens before
 *     any launch; on error nothing is enqueued and csa2_last_error() (a
 *     thread-local string) says why.  No exceptions cross the ABI.
 *   - Outputs must not overlap inputs.  Calls on distinct streams are
 *     thread-safe.  The library's only mutable global state is a set of
 *     per-device, set-once flags and addresses (kernel LDS limits, the
 *     location of csa2_sparse_attn_decode_noalloc's scratch array), that
 *     scratch array itself, which is shared by every call of that one entry
 *     point on a device (see there), and the benchmark timing hook of
 *     csa2_set_launch_events (unset unless a caller sets it).
 *   - Results are bitwise deterministic for fixed inputs and launch shapes.
 *   - bf16 values are passed as uint16_t bit patterns.
 *
 * Fixed dimensions ([KVC] 1 setup list): main latent 512, 64 attention
 * heads of width 512, 32 indexer heads of width 128, window <= 128.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t csa2_status;
enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum, overlap */
  CSA2_ERR_UNSUPPORTED = 2, /* k or block outside the supported range     */
  CSA2_ERR_ALIGNMENT = 3,   /* a pointer is not aligned as documented     */
  CSA2_ERR_WORKSPACE = 4,   /* workspace missing or too small             */
  CSA2_ERR_HIP = 5          /* a HIP runtime call failed (e.g. no device) */
};

/* Cache entry formats. */
enum {
  /* Main KV, [KVC] 5 and [ARCH] 2.4.4: 512 channels as E2M1 codes with one
   * E4M3 scale per 16 channels, s_g = E4M3(max|x| / 6), x_i -> E2M1(x_i /
   * s_g); rounding to nearest, ties to even, saturating; sign of zero kept.
   * Row = 256 code bytes (channel 2i in the low nibble of byte i, 2i+1 in
   * the high nibble) in one plane and 32 scale bytes in another: 288 B per
   * entry ([KVC] 2, b_main equation). */
  CSA2_FMT_MAIN = 0,
  /* Indexer key, [KVC] 2 and [ARCH] 2.4.4: 128 elements as OCP MXFP4 --
   * E2M1 codes with one E8M0 scale per 32, exponent floor(log2 max|x|) - 2
   * clamped to [-127, 127] (an all-zero block stores code 0).  Row = 64
   * code bytes + 4 scale bytes: 68 B per entry. */
  CSA2_FMT_IDX = 1,
  /* Sliding-window KV, kept in FP8 ([ARCH] 2.4.4): 512 unscaled E4M3 bytes
   * per row; no scale plane. */
  CSA2_FMT_SWA = 2
};

/* Key format of csa2_indexer_score. */
enum {
  CSA2_KEYS_MXFP4 = 0, /* CSA2_FMT_IDX planes                            */
  CSA2_KEYS_BF16 = 1   /* bf16 rows of 128 (the pooled block keys)        */
};

/* Operations for csa2_workspace_size. */
enum {
  CSA2_OP_TOPK = 0,
  CSA2_OP_DECODE = 1, /* csa2_sparse_attn_decode                          */
  CSA2_OP_REUSE = 2,  /* csa2_reuse_attn                                  */
  CSA2_OP_FULL_POOL = 3, /* csa2_full_pool_decode (needs the pool options)  */
  CSA2_OP_REINDEX = 4,   /* csa2_reindex_decode (n_cap argument = n_pool)  */
  CSA2_OP_COMPRESS = 5   /* csa2_compress_append (n_cap = m, k = d)        */
};

/* The caches one Full layer owns (or a Reindex layer shares). */
typedef struct {
  const uint8_t *main_codes;   /* [B][n_cap][256], 16-byte aligned         */
  const uint8_t *main_scales;  /* [B][n_cap][32],  4-byte aligned          */
  const uint8_t *idx_codes;    /* [B][n_cap][64],  16-byte aligned         */
  const uint8_t *idx_scales;   /* [B][n_cap][4],   4-byte aligned          */
  const uint16_t *block_keys;  /* [B][ceil(n_cap/block)][128] bf16, or
                                  NULL when no pool is used; 16-B aligned  */
  int64_t n_cap;               /* entry capacity per sequence              */
  const int32_t *n_entries;    /* [B] visible entries per sequence (device)*/
} csa2_cache;

/* Hierarchical candidate pool ([KVC] 4.3, [ARCH] 2.3.2): keep the top
 * min(n_blocks_keep, blocks) blocks of `block` positions by block score and
 * score only their positions. */
typedef struct {
  int32_t n_blocks_keep; /* e.g. 2048 */
  int32_t block;         /* e.g. 8    */
} csa2_pool_opts;

/* ------------------------------------------------------------------------
 * csa2_pack_kv -- quantise float32 rows into a cache format (the write
 * path; [KVC] 5 quantiser equation for CSA2_FMT_MAIN).
 *   fmt        CSA2_FMT_MAIN / _IDX / _SWA
 *   src        [n_rows][512 or 128] float32, finite values
 *   dst_codes  [n_rows][256 / 64 / 512] bytes (16-byte aligned)
 *   dst_scales [n_rows][32 / 4] bytes; must be NULL for CSA2_FMT_SWA
 * Bit-exact with the oracle.  n_rows == 0 is a no-op. */
csa2_status csa2_pack_kv(int32_t fmt, const float *src, int64_t n_rows,
                         void *dst_codes, void *dst_scales, void *stream);

/* csa2_unpack_kv -- exact dequantisation of packed rows to float32
 * (E2M1 x E4M3, E2M1 x 2^(E8M0-127), or E4M3), for checking. */
csa2_status csa2_unpack_kv(int32_t fmt, const void *codes, const void *scales,
                           int64_t n_rows, float *dst, void *stream);

/* csa2_build_block_keys -- pooled block keys for the hierarchical first
 * stage: key of block j of sequence b = bf16 (round to nearest even, once)
 * of the exact mean of the dequantised indexer keys at positions
 * block*j .. block*j+block-1 that are < n_entries[b]; blocks past the end
 * are written as zeros.
 *   idx_codes/idx_scales  [B][n_cap] CSA2_FMT_IDX planes
 *   block_keys            [B][ceil(n_cap/block)][128] bf16 out
 *   block                 1..64 */
csa2_status csa2_build_block_keys(const uint8_t *idx_codes,
                                  const uint8_t *idx_scales, int64_t n_cap,
                                  const int32_t *n_entries, int32_t B,
                                  int32_t block, uint16_t *block_keys,
                                  void *stream);

/* ------------------------------------------------------------------------
 * csa2_indexer_score -- lightning-indexer scores ([V4] CSA step 2 score
 * equation; [KVC] 4.1):  I_j = sum_{h<32} w_h * ReLU(q_h . K_j).
 *   keyfmt    CSA2_KEYS_MXFP4: k_codes [B][n_cap][64], k_scales [B][n_cap][4]
 *             CSA2_KEYS_BF16:  k_codes bf16 [B][n_cap][128], k_scales NULL
 *   n_entries [B] valid rows per sequence (device)
 *   cand      NULL: score rows 0..n_cap-1 into scores[B][n_cap];
 *             else [B][n_cand] row ids to score into scores[B][n_cand]
 *   q_idx     [B][32][128] bf16; w [B][32] float32
 *   n_cap     <= 2^24 (CSA2_ERR_UNSUPPORTED beyond)
 * Rows >= n_entries[b] (or ids outside [0, n_entries[b])) get -inf.
 * Products are exact (bf16 x dequantised FP4); accumulation is float32. */
csa2_status csa2_indexer_score(int32_t keyfmt, const void *k_codes,
                               const void *k_scales, int64_t n_cap,
                               const int32_t *n_entries, const int32_t *cand,
                               int32_t n_cand, const uint16_t *q_idx,
                               const float *w, int32_t B, float *scores,
                               void *stream);

/* csa2_indexer_score_fp4q -- the same scores with the indexer query itself
 * in OCP MXFP4, as V4 trains it for FP4 scoring ([ARCH] 2.4.4; [KVC] 5):
 *   q_codes   [B][32][64] E2M1 codes (16-byte aligned), q_scales [B][32][4]
 *             E8M0: the CSA2_FMT_IDX planes of the 32 query heads (what
 *             csa2_pack_kv(CSA2_FMT_IDX, q, 32 * B, ...) writes)
 *   other arguments as in csa2_indexer_score.
 * I_j = sum_h w_h * ReLU(deq(q_h) . K_j).  MXFP4 keys are scored from the
 * FP4 codes directly (E2M1 x E2M1 products with their two scales: exact);
 * bf16 keys against the exactly dequantised query.  Accumulation is
 * float32. */
csa2_status csa2_indexer_score_fp4q(int32_t keyfmt, const void *k_codes,
                                    const void *k_scales, int64_t n_cap,
                                    const int32_t *n_entries,
                                    const int32_t *cand, int32_t n_cand,
                                    const uint8_t *q_codes,
                                    const uint8_t *q_scales, const float *w,
                                    int32_t B, float *scores, void *stream);

/* ------------------------------------------------------------------------
 * csa2_topk -- exact top-k per row ([V4] CSA step 2 top-k equation; [KVC]
 * 4.1 S_t = Top512).  Row b holds scores[b*ld + i], i < n_valid[b]
 * (n_valid NULL: ld).  Entries that are -inf or NaN, or whose id is < 0,
 * are never chosen.  Order: higher score first, equal scores by lower id,
 * where id = ids[b*ld + i] (ids NULL: id = i; ids must increase with i
 * among valid entries).  Output out[b][k*block]: the chosen ids in
 * ascending order; with block > 1 each chosen id j is expanded to the
 * positions block*j .. block*j+block-1 that are < limit[b] (limit NULL: no
 * bound) -- the pool expansion of [KVC] 4.3.  Unused slots hold -1.
 *   k in 1..2048, block in 1..64, ld >= 1.
 *   ws / ws_bytes: workspace of csa2_workspace_size(CSA2_OP_TOPK, B, ld,
 *   k, NULL) bytes, 256-byte aligned. */
csa2_status csa2_topk(const float *scores, int64_t ld, const int32_t *n_valid,
                      const int32_t *ids, int32_t B, int32_t k, int32_t block,
                      const int32_t *limit, int32_t *out, void *ws,
                      size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn_decode -- one decode query per sequence through a Full
 * (or, pointed at shared caches, Reindex) CSA2 layer ([ARCH] 2.3.1; [KVC]
 * 4.1 and 4.2 table):
 *   scores over the n_entries[b] visible entries (or, with `pool`, the
 *   hierarchical pool of [KVC] 4.3), top-k, then
 *   o_h = softmax(scale * q_h K^T) K over the chosen main entries followed
 *   by the first n_swa[b] window rows (keys double as values, [V4] CSA
 *   step 3).
 *   kv        caches (kv->block_keys required when pool != NULL)
 *   q_idx     [B][32][128] bf16, w [B][32] float32 (indexer query/weights)
 *   q         [B][64][512] bf16 attention queries (16-byte aligned)
 *   swa       [B][128][512] E4M3 window rows; n_swa [B] (device, <= 128)
 *   k         1..2048 (512 in the pages)
 *   out       [B][64][512] bf16 (16-byte aligned)
 *   topk_out  [B][k] chosen ids ascending, -1 padded (for Reuse layers)
 *   n_cap     <= 2^24 here (CSA2_ERR_UNSUPPORTED beyond)
 * Keys/values are dequantised exactly (to fp16); logits, softmax and
 * accumulation are float32; probabilities enter the P.V product as fp16.
 * The query products run in fp16 too: each head's bf16 query is first
 * scaled by a power of two that brings its largest |q| into [2^14, 2^15)
 * (the logit scale takes the inverse), so every value within 2^28 of the
 * head's largest converts exactly and none overflows.  Supported: max |q|
 * per head below 2^79 (the prescale exponent is clamped to [-100, 64]);
 * beyond that the output is undefined.  The same holds for every call that
 * runs the attention (reuse, full-pool, reindex, the _ex and _fp4q
 * variants). */
csa2_status csa2_sparse_attn_decode(const csa2_cache *kv,
                                    const uint16_t *q_idx, const float *w,
                                    const uint16_t *q, const uint8_t *swa,
                                    const int32_t *n_swa, int32_t B, int32_t k,
                                    float scale, const csa2_pool_opts *pool,
                                    uint16_t *out, int32_t *topk_out, void *ws,
                                    size_t ws_bytes, void *stream);

/* csa2_sparse_attn_decode_noalloc -- csa2_sparse_attn_decode for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same call without a
 * workspace.  Its scratch is a fixed array inside the library, one copy per
 * GPU, of CSA2_NOALLOC_SCRATCH_BYTES; the library looks up the current
 * device's copy on the first call on that device and allocates nothing,
 * ever.  A call whose workspace (csa2_workspace_size(CSA2_OP_DECODE, B,
 * n_cap, k, pool)) exceeds the array fails with CSA2_ERR_WORKSPACE and
 * enqueues nothing: 32 MiB covers 32 sequences of 32,768 entries at
 * k = 512.  Every call on a GPU uses the same array, so calls that overlap
 * on one GPU (on different streams, or from different threads) race and
 * must be ordered by the caller; nothing in it needs to start at zero.
 * Arguments, outputs and errors otherwise as csa2_sparse_attn_decode. */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
csa2_status csa2_sparse_attn_decode_noalloc(
    const csa2_cache *kv, const uint16_t *q_idx, const float *w,
    const uint16_t *q, const uint8_t *swa, const int32_t *n_swa, int32_t B,
    int32_t k, float scale, const csa2_pool_opts *pool, uint16_t *out,
    int32_t *topk_out, void *stream);

/* csa2_sparse_attn_decode_fp4q -- csa2_sparse_attn_decode with the
 * indexer query in MXFP4 planes (q_codes [B][32][64], q_scales [B][32][4],
 * as in csa2_indexer_score_fp4q); every other argument, the workspace and
 * the outputs as there. */
csa2_status csa2_sparse_attn_decode_fp4q(
    const csa2_cache *kv, const uint8_t *q_codes, const uint8_t *q_scales,
    const float *w, const uint16_t *q, const uint8_t *swa,
    const int32_t *n_swa, int32_t B, int32_t k, float scale,
    const csa2_pool_opts *pool, uint16_t *out, int32_t *topk_out, void *ws,
    size_t ws_bytes, void *stream);

/* csa2_full_pool_decode -- the first Full layer of a hierarchical decoder
 * group as the pages define it ([KVC] 4.3 equation; [ARCH] 2.3.2 and
 * Figure 5): exactly csa2_sparse_attn_decode without a pool (scores over
 * all n_entries[b] visible entries, its own top-k, attention), and besides
 * it the candidate pool of the Reindex layers after it -- block j (positions
 * 8j .. 8j+7) scores the largest of its fine scores, the n_blocks_keep
 * best blocks (equal maxima: the lower block first) are taken and expanded
 * to their positions below n_entries[b].
 *   pool      n_blocks_keep in 1..2048, block == 8 (CSA2_ERR_UNSUPPORTED
 *             otherwise); kv->block_keys is not used
 *   pool_out  [B][n_blocks_keep * 8] positions, ascending, -1 padded
 *   other arguments and outputs as in csa2_sparse_attn_decode.
 *   ws / ws_bytes: csa2_workspace_size(CSA2_OP_FULL_POOL, B, n_cap, k,
 *             pool) bytes, 256-byte aligned. */
csa2_status csa2_full_pool_decode(const csa2_cache *kv, const uint16_t *q_idx,
                                  const float *w, const uint16_t *q,
                                  const uint8_t *swa, const int32_t *n_swa,
                                  int32_t B, int32_t k, float scale,
                                  const csa2_pool_opts *pool, uint16_t *out,
                                  int32_t *topk_out, int32_t *pool_out,
                                  void *ws, size_t ws_bytes, void *stream);

/* csa2_reindex_decode -- a Reindex-mode layer ([KVC] 4.2 table, 4.3
 * equation; [ARCH] 2.3.1): the layer's own indexer query (q_idx, w) scores
 * only the pool positions on the shared indexer keys, its top-k among them
 * is taken (ids ascending, -1 padded), then attention over those main
 * entries plus the layer's own window, as in csa2_sparse_attn_decode.
 *   pool      [B][n_pool] positions (from csa2_full_pool_decode); entries
 *             < 0 or >= n_entries[b] are skipped; valid entries ascending
 *   n_pool    1..2^26
 *   ws / ws_bytes: csa2_workspace_size(CSA2_OP_REINDEX, B, n_pool, k,
 *             NULL) bytes, 256-byte aligned. */
csa2_status csa2_reindex_decode(const csa2_cache *kv, const int32_t *pool,
                                int64_t n_pool, const uint16_t *q_idx,
                                const float *w, const uint16_t *q,
                                const uint8_t *swa, const int32_t *n_swa,
                                int32_t B, int32_t k, float scale,
                                uint16_t *out, int32_t *topk_out, void *ws,
                                size_t ws_bytes, void *stream);

/* csa2_reuse_attn -- a Reuse-mode layer ([ARCH] 2.3.1; [KVC] 4.2 table):
 * no indexer; attention over the given top-k ids (entries < 0 skipped) of
 * the shared main cache plus this layer's own window.  Arguments as in
 * csa2_sparse_attn_decode; topk [B][k]. */
csa2_status csa2_reuse_attn(const uint8_t *main_codes,
                            const uint8_t *main_scales, int64_t n_cap,
                            const int32_t *topk, int32_t k, const uint16_t *q,
                            const uint8_t *swa, const int32_t *n_swa,
                            int32_t B, float scale, uint16_t *out, void *ws,
                            size_t ws_bytes, void *stream);

/* csa2_attn_opts -- the attention details of [V4] "other details" (NULL
 * pointers leave either out):
 *   sink        [64] float32 per-head sink logits z'_h (attention-sink
 *               equation): exp(z'_h) joins only the softmax denominator, in
 *               the units of the scaled logits scale * q.k
 *   pos         [B] int32 query positions t (device): the last 64 output
 *               dims are de-rotated by -t (partial-RoPE paragraph, the
 *               R_{-t} o_t equation).  Reading: interleaved pairs
 *               (448 + 2i, 449 + 2i), frequency rope_theta^(-2i/64),
 *               position p turning (x, y) into (x cos - y sin, x sin + y cos)
 *               of the angle p * frequency
 *   rope_theta  > 0 (10000 in the usual RoPE), used with pos. */
typedef struct {
  const float *sink;
  const int32_t *pos;
  float rope_theta;
} csa2_attn_opts;

/* csa2_sparse_attn_decode_ex / csa2_reuse_attn_ex -- csa2_sparse_attn_decode
 * and csa2_reuse_attn with the csa2_attn_opts details applied to the
 * output (opts NULL: identical to the plain calls). */
csa2_status csa2_sparse_attn_decode_ex(const csa2_cache *kv,
                                       const uint16_t *q_idx, const float *w,
                                       const uint16_t *q, const uint8_t *swa,
                                       const int32_t *n_swa, int32_t B,
                                       int32_t k, float scale,
                                       const csa2_pool_opts *pool,
                                       const csa2_attn_opts *opts,
                                       uint16_t *out, int32_t *topk_out,
                                       void *ws, size_t ws_bytes,
                                       void *stream);
csa2_status csa2_reuse_attn_ex(const uint8_t *main_codes,
                               const uint8_t *main_scales, int64_t n_cap,
                               const int32_t *topk, int32_t k,
                               const uint16_t *q, const uint8_t *swa,
                               const int32_t *n_swa, int32_t B, float scale,
                               const csa2_attn_opts *opts, uint16_t *out,
                               void *ws, size_t ws_bytes, void *stream);

/* csa2_sparse_attn_decode_fp4q_ex / csa2_full_pool_decode_ex /
 * csa2_reindex_decode_ex -- the MXFP4-query decode and the two layer calls
 * of the hierarchical decoder group with the same csa2_attn_opts details
 * ([V4] 2.3 other details: they apply to every CSA head); opts NULL:
 * identical to the plain calls, whose arguments, workspaces and outputs
 * they share. */
csa2_status csa2_sparse_attn_decode_fp4q_ex(
    const csa2_cache *kv, const uint8_t *q_codes, const uint8_t *q_scales,
    const float *w, const uint16_t *q, const uint8_t *swa,
    const int32_t *n_swa, int32_t B, int32_t k, float scale,
    const csa2_pool_opts *pool, const csa2_attn_opts *opts, uint16_t *out,
    int32_t *topk_out, void *ws, size_t ws_bytes, void *stream);
csa2_status csa2_full_pool_decode_ex(
    const csa2_cache *kv, const uint16_t *q_idx, const float *w,
    const uint16_t *q, const uint8_t *swa, const int32_t *n_swa, int32_t B,
    int32_t k, float scale, const csa2_pool_opts *pool,
    const csa2_attn_opts *opts, uint16_t *out, int32_t *topk_out,
    int32_t *pool_out, void *ws, size_t ws_bytes, void *stream);
csa2_status csa2_reindex_decode_ex(
    const csa2_cache *kv, const int32_t *pool, int64_t n_pool,
    const uint16_t *q_idx, const float *w, const uint16_t *q,
    const uint8_t *swa, const int32_t *n_swa, int32_t B, int32_t k,
    float scale, const csa2_attn_opts *opts, uint16_t *out,
    int32_t *topk_out, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_compress_append -- the CSA2 write path at decode time ([KVC] 4.1
 * main-KV, sequence-compression and indexer-K equations; [ARCH] 2.3):
 * for each sequence the hidden states of the m newest tokens give
 * C = H W^KV and Z = H W^Z (512 wide); the new main entry is their
 * per-channel softmax(Z)-weighted sum over the m tokens, C_bar (blocks
 * without overlap), and its indexer key K^I = C_bar W^IK (128 wide).  C_bar
 * is packed (CSA2_FMT_MAIN rules, bit-exact with csa2_pack_kv of the same
 * float32 values) into row rows[b] of the main planes and K^I (CSA2_FMT_IDX)
 * into the same row of the indexer planes; rows outside [0, n_cap) are not
 * written.  With swa non-NULL each token's C_i is also written, E4M3, to
 * window slot (swa_slot[b] + i) mod 128.
 *   h           [B][m][d] bf16 (16-byte aligned); d a multiple of 16,
 *               16..16384; m 1..16
 *   w_kv, w_z   [512][d] bf16 (output x input, 16-byte aligned)
 *   w_ik        [128][512] bf16 (16-byte aligned)
 *   rows        [B] int32 (device): the cache row of each new entry
 *   main_codes/main_scales/idx_codes/idx_scales: the caches [B][n_cap][...]
 *   swa, swa_slot  [B][128][512] window rows and [B] int32 slots, or both
 *               NULL
 *   cbar_out [B][512], ki_out [B][128], c_out [B][m][512]: optional float32
 *               copies of C_bar, K^I and C (NULL to skip)
 *   ws / ws_bytes: csa2_workspace_size(CSA2_OP_COMPRESS, B, m, d, NULL)
 *               bytes, 256-byte aligned.
 * Products are exact (bf16); sums are float32 in a fixed order. */
csa2_status csa2_compress_append(const uint16_t *h, int32_t B, int32_t m,
                                 int32_t d, const uint16_t *w_kv,
                                 const uint16_t *w_z, const uint16_t *w_ik,
                                 const int32_t *rows, uint8_t *main_codes,
                                 uint8_t *main_scales, uint8_t *idx_codes,
                                 uint8_t *idx_scales, int64_t n_cap,
                                 uint8_t *swa, const int32_t *swa_slot,
                                 float *cbar_out, float *ki_out, float *c_out,
                                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Helpers. */

/* Workspace bytes an operation needs (0 on bad arguments).  For
 * CSA2_OP_TOPK `n_cap` is the row length ld. */
size_t csa2_workspace_size(int32_t op, int32_t B, int64_t n_cap, int32_t k,
                           const csa2_pool_opts *pool);

/* Bytes per cache entry of a format (288, 68, 512), -1 on a bad format. */
int32_t csa2_entry_bytes(int32_t fmt);

/* Global-KV bytes per token ([KVC] 2, B_global equation): sum over the
 * layers that produce KV of (main + indexer entry bytes) / m_l, given each
 * such layer's compression ratio m_l.  For the V4.1 plan {2, 2, 2, 1} this
 * is 890. */
double csa2_kv_bytes_per_token(const int32_t *m_of_kv_layers, int32_t n);

/* Per-kernel timing hook for benchmarks (not part of the method).  While set
 * (n > 0), each call of csa2_sparse_attn_decode(_fp4q/_ex/_noalloc) and
 * csa2_reuse_attn(_ex) records events[0] on its stream just before its first
 * kernel and events[i] right after its i-th kernel, for i < n (further
 * kernels of the call record nothing), so the time between consecutive
 * events is one kernel of that call as it runs inside the step.  The events
 * are the caller's hipEvent_t handles (created with timing enabled and
 * owned by the caller).  Process-wide setting, for single-threaded
 * benchmarking only: set it, make one call, set the next events or clear
 * with n = 0.  Returns CSA2_ERR_INVALID_ARG for n < 0, n > 16 or a null
 * array with n > 0; a failed record makes the call return CSA2_ERR_HIP. */
csa2_status csa2_set_launch_events(void *const *events, int32_t n);

/* Events recorded by the latest call made while csa2_set_launch_events was
 * set (its kernel count + 1 when enough events were given). */
int32_t csa2_launch_events_recorded(void);

/* Thread-local message of the last failed call on this thread. */
const char *csa2_last_error(void);

/* Library version string. */
const char *csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
