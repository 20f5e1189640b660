"""Oracle for the decode path of one CSA2 layer: cache packing, the lightning
indexer, exact top-k, the hierarchical candidate pool, and shared-latent
multi-query attention over the selected entries plus the sliding window.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 NumPy.  It shares no code
with the GPU library and imports nothing from it; only tests/, the smoke
check and the CPU-baseline leg of the benchmark may call it.

Sources (web pages, cited by title):
  [KVC]  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
         (mer.run post): section 2 (entry sizes), 4.1 (single-layer
         formulas), 4.2 (Full / Reindex / Reuse table), 4.3 (hierarchical
         indexer equation), 5 (FP4 quantiser equation).
  [ARCH] "DeepSeek-V4.1-Flash, 2. Architecture" course notes: 2.3 (CSA2),
         2.3.1 (mode definitions, Figure 4), 2.3.2 (hierarchical sparse
         indexer, Figure 5), 2.4.4 (FP4 main KV cache).
  [V4]   "DeepSeek-V4: Towards Highly Efficient Million-Token Context
         Intelligence" (baisen.site): CSA step 2 (index score and top-k
         equations), CSA step 3 (shared-KV MQA equation).

Layouts (identical on both sides; a library definition the pages leave
open): a main entry is 256 code bytes then 32 scale bytes; channel 2i sits in
the low nibble of code byte i and channel 2i+1 in the high nibble; scale
byte g covers channels 16g..16g+15.  An indexer entry is 64 code bytes and 4
E8M0 bytes, same nibble order, scale byte g for elements 32g..32g+31.
A sliding-window row is 512 unscaled E4M3 bytes.

Parity pins for every function here live in tests/test_oracle_*.py.
"""
import numpy as np

from . import formats as F

D_MAIN = 512          # main-KV latent width            [KVC] 1 setup list
D_IDX = 128           # indexer head dim                [KVC] 1 setup list
H_IDX = 32            # indexer heads                   [KVC] 1 setup list
H_ATTN = 64           # attention query heads           [KVC] 1 setup list
G_MAIN = 16           # channels per E4M3 scale         [KVC] 2, 5
G_IDX = 32            # elements per E8M0 scale         [KVC] 2
N_WIN = 128           # sliding-window length           [KVC] 1, 4.1


# ------------------------------------------------------------ packing ----
def _pack_nibbles(codes):
    """[..., 2m] 4-bit codes -> [..., m] bytes, even element in low nibble."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _unpack_nibbles(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def pack_main(x):
    """FP4 main-KV quantiser, [KVC] 5 and [ARCH] 2.4.4.

    For each 16-channel group g: s_g = E4M3(max_i |x_i| / 6), then each
    channel is E2M1(x_i / s_g) with the decoded s_g.  A group whose scale
    rounds to zero stores sign-only zero codes.
    x: float32 [n, 512] -> (codes uint8 [n, 256], scales uint8 [n, 32]).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = x.shape[0]
    g = x.reshape(n, D_MAIN // G_MAIN, G_MAIN)
    amax = np.abs(g).max(axis=-1)
    s_code = F.e4m3_encode(amax / 6.0)
    s = F.e4m3_decode(s_code)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s > 0, g / np.where(s > 0, s, 1.0), 0.0 * g)
    codes = F.e2m1_encode(np.where(s > 0, r, np.copysign(0.0, g)))
    return _pack_nibbles(codes.reshape(n, D_MAIN)), s_code.astype(np.uint8)


def unpack_main(codes, scales):
    """Dequantise main entries: E2M1(code) * E4M3(scale), exact in float64."""
    v = F.e2m1_decode(_unpack_nibbles(codes))                  # [n, 512]
    s = F.e4m3_decode(scales)                                  # [n, 32]
    n = v.shape[0]
    return (v.reshape(n, -1, G_MAIN) * s[..., None]).reshape(n, D_MAIN)


def pack_idx(x):
    """OCP MXFP4 indexer key, [KVC] 2 and [ARCH] 2.4.4 (the MX rule itself is
    the OCP Microscaling v1.0 definition the pages name).

    Per 32-element block: shared exponent e = floor(log2(max|x|)) - 2
    (2 = largest E2M1 exponent), clamped to the E8M0 range [-127, 127],
    stored as e + 127; elements are E2M1(x / 2**e), saturating at 6.  An
    all-zero block stores scale code 0 and sign-only zero elements.
    x: float32 [n, 128] -> (codes uint8 [n, 64], scales uint8 [n, 4]).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = x.shape[0]
    blk = x.reshape(n, D_IDX // G_IDX, G_IDX)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex - 1 - 2, -127, 127)
    e = np.where(amax > 0, e, -127)
    r = blk / np.exp2(e)[..., None]
    codes = F.e2m1_encode(r)
    return (_pack_nibbles(codes.reshape(n, D_IDX)),
            (e + 127).astype(np.uint8))


def unpack_idx(codes, scales):
    v = F.e2m1_decode(_unpack_nibbles(codes))
    s = F.e8m0_decode(scales)
    n = v.shape[0]
    return (v.reshape(n, -1, G_IDX) * s[..., None]).reshape(n, D_IDX)


def pack_swa(x):
    """Sliding-window KV kept in FP8 ([ARCH] 2.4.4, [KVC] 5): one unscaled
    E4M3 byte per value (the pages give no scale for it)."""
    return F.e4m3_encode(np.asarray(x, dtype=np.float32).astype(np.float64))


def unpack_swa(codes):
    return F.e4m3_decode(codes)


def block_keys(idx_codes, idx_scales, n_entries, block=8):
    """Pooled block keys for the hierarchical indexer's first stage.

    Block b holds positions block*b .. block*b+block-1 that are < n_entries;
    its key is the mean of the dequantised indexer keys present, rounded
    once to bfloat16 (the sum of at most 8 such values is exact in float64).
    Returns uint16 bf16 bits [ceil(n_entries / block), 128].
    """
    k = unpack_idx(idx_codes[:n_entries], idx_scales[:n_entries])
    nb = -(-n_entries // block)
    pad = nb * block - n_entries
    kp = np.concatenate([k, np.zeros((pad, D_IDX))], axis=0)
    sums = kp.reshape(nb, block, D_IDX).sum(axis=1)
    cnt = np.full(nb, float(block))
    cnt[-1] = block - pad
    return F.bf16_round(sums / cnt[:, None])


# ------------------------------------------------------------ indexer ----
def indexer_scores(q_idx_bits, w, keys):
    """Lightning-indexer score, [V4] CSA step 2 and [KVC] 4.1:
        I_j = sum_h w_h * ReLU(q_h . K_j)
    q_idx_bits: bf16 bits [32, 128]; w: [32]; keys: float64 [n, 128]
    (dequantised).  Returns float64 [n]."""
    q = F.bf16_bits_to_f64(q_idx_bits)
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    dots = keys @ q.T                                          # [n, 32]
    return np.maximum(dots, 0.0) @ w


def indexer_scores_fp4q(q_codes, q_scales, w, keys):
    """The lightning-indexer score with the query itself in MXFP4: [ARCH]
    2.4.4 (V4 trains the indexer query and key for FP4 scoring, in OCP
    MXFP4; [KVC] 5 says the same).  The query heads are packed like an
    indexer key (pack_idx of the 32 rows) and scored dequantised:
        I_j = sum_h w_h * ReLU(deq(q_h) . K_j)
    q_codes uint8 [32, 64], q_scales uint8 [32, 4]; w [32]; keys float64
    [n, 128] (dequantised).  Returns float64 [n]."""
    q = unpack_idx(q_codes, q_scales)
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    dots = keys @ q.T                                          # [n, 32]
    return np.maximum(dots, 0.0) @ w


def topk(scores, k, ids=None):
    """Exact top-k, [V4] CSA step 2 / [KVC] 4.1 (S_t = Top512 of I_t).

    Order: higher score first, equal scores by lower id (the pages give no
    tie rule).  Returns the chosen ids sorted ascending, padded with -1 to
    length k.  `ids` (default 0..n-1) are the ids reported for the scores.
    """
    s = np.asarray(scores, dtype=np.float64)
    ids = np.arange(len(s)) if ids is None else np.asarray(ids)
    order = np.lexsort((ids, -s))
    chosen = np.sort(ids[order[:min(k, len(s))]])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(chosen)] = chosen
    return out


def topk_gap(scores, k):
    """Relative gap between the k-th and (k+1)-th largest scores
    ((s_k - s_k+1) / s_k); +inf when fewer than k+1 scores exist."""
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    if len(s) <= k:
        return np.inf
    return (s[k - 1] - s[k]) / abs(s[k - 1]) if s[k - 1] != 0 else (
        np.inf if s[k] < s[k - 1] else 0.0)


def hier_pool(block_scores, n_entries, n_keep=2048, block=8):
    """Candidate pool of the hierarchical indexer ([KVC] 4.3 equation,
    [ARCH] 2.3.2): keep the top min(n_keep, n_blocks) blocks by block score
    and take the union of their positions (< n_entries), ascending.
    Returned padded with -1 to n_keep * block."""
    nb = len(block_scores)
    blocks = topk(block_scores, min(n_keep, nb))
    blocks = blocks[blocks >= 0]
    pos = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    pos = pos[pos < n_entries]
    out = np.full(n_keep * block, -1, dtype=np.int64)
    out[:len(pos)] = pos
    return out


def block_max_scores(scores, n_entries, block=8):
    """Block score of the hierarchical indexer as the pages define it,
    [KVC] 4.3 equation and [ARCH] 2.3.2: s_b = max of the first Full
    layer's fine scores I_j over the positions j < n_entries of block b.
    Returns float64 [ceil(n_entries / block)]."""
    nb = -(-n_entries // block)
    pad = np.full(nb * block, -np.inf)
    pad[:n_entries] = np.asarray(scores[:n_entries], dtype=np.float64)
    return pad.reshape(nb, block).max(axis=1)


# ---------------------------------------------------------- attention ----
def mqa_decode(q_bits, keys, scale):
    """Shared-KV multi-query attention for one decode query, [V4] CSA step 3
    and [KVC] 4.1: o_h = softmax(q_h K^T * scale) K, every key doubling as
    its value.  q_bits: bf16 bits [64, 512]; keys float64 [m, 512].
    Softmax with the row maximum subtracted; float64 throughout."""
    q = F.bf16_bits_to_f64(q_bits)
    logits = (q @ keys.T) * float(scale)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ keys


def mqa_decode_sink(q_bits, keys, scale, sink):
    """mqa_decode with a per-head attention sink, [V4] "other details",
    attention-sink equation: a learnable logit z'_h joins only the softmax
    denominator, a_s = exp(l_s) / (sum_s' exp(l_s') + exp(z'_h)), so a head's
    weights may sum to less than 1.  sink: [64] (logit units, like
    q.k * scale).  float64 throughout."""
    q = F.bf16_bits_to_f64(q_bits)
    z = np.asarray(sink, dtype=np.float32).astype(np.float64)
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], keys.shape[1]))
    logits = (q @ keys.T) * float(scale)                     # [64, m]
    ref = np.maximum(logits.max(axis=1), z)
    p = np.exp(logits - ref[:, None])
    den = p.sum(axis=1) + np.exp(z - ref)
    return (p / den[:, None]) @ keys


def rope_derotate(o, t, theta=10000.0, r=64):
    """The output de-rotation of partial RoPE, [V4] "other details" (partial
    RoPE paragraph and the R_{-t} o_t equation): RoPE applies to the last
    r = 64 dims only, and the output is rotated once by position -t so the
    absolute rotation R_s carried by each value becomes R_{s-t}.  Reading
    (the page does not spell the rotation out): standard RoPE on the
    interleaved pairs (d0 + 2i, d0 + 2i + 1), d0 = 512 - r, with frequency
    theta ** (-2i / r); position p maps (x, y) to
    (x cos p w - y sin p w, x sin p w + y cos p w).  o: [H, 512]."""
    o = np.array(o, dtype=np.float64)
    d0 = o.shape[1] - r
    i = np.arange(r // 2)
    ang = -float(t) * float(theta) ** (-2.0 * i / r)
    c, s = np.cos(ang), np.sin(ang)
    x, y = o[:, d0::2].copy(), o[:, d0 + 1::2].copy()
    o[:, d0::2] = x * c - y * s
    o[:, d0 + 1::2] = x * s + y * c
    return o


def gather_keys(main_codes, main_scales, idx, swa_codes, n_swa):
    """Keys of one query: the selected main entries (ids >= 0, in the given
    order) followed by the first n_swa sliding-window rows, concatenated
    without de-duplication ([KVC] 4.1 attention line)."""
    sel = np.asarray(idx)
    sel = sel[sel >= 0]
    km = unpack_main(main_codes[sel], main_scales[sel])
    ks = unpack_swa(swa_codes[:n_swa])
    return np.concatenate([km, ks], axis=0)


# --------------------------------------------------------- whole layer ---
def full_layer(main_codes, main_scales, idx_codes, idx_scales, n_entries,
               q_idx_bits, w, q_bits, swa_codes, n_swa, k, scale):
    """Decode of one Full-mode (or Reindex-mode, on shared caches) layer for
    one sequence, [ARCH] 2.3.1 and [KVC] 4.2 table: score every visible
    entry, take the top-k, attend over it plus the window.
    Returns (top-k ids [k], output float64 [64, 512], scores [n])."""
    keys = unpack_idx(idx_codes[:n_entries], idx_scales[:n_entries])
    sc = indexer_scores(q_idx_bits, w, keys)
    sel = topk(sc, k)
    kv = gather_keys(main_codes, main_scales, sel, swa_codes, n_swa)
    return sel, mqa_decode(q_bits, kv, scale), sc


def reuse_layer(main_codes, main_scales, sel, q_bits, swa_codes, n_swa,
                scale):
    """Reuse-mode layer, [ARCH] 2.3.1 and [KVC] 4.2 table: no indexer, the
    given (latest) top-k ids, own query and own window."""
    kv = gather_keys(main_codes, main_scales, sel, swa_codes, n_swa)
    return mqa_decode(q_bits, kv, scale)


def hier_layer(main_codes, main_scales, idx_codes, idx_scales, bkeys_bits,
               n_entries, q_idx_bits, w, q_bits, swa_codes, n_swa, k, scale,
               n_keep=2048, block=8):
    """Hierarchical decode: block scores on pooled bf16 block keys, the
    top-n_keep block pool, fine scores on the pool only, top-k inside the
    pool reported as sequence positions, then attention.
    Returns (top-k ids, output, pool, pool scores)."""
    bs = indexer_scores(q_idx_bits, w, F.bf16_bits_to_f64(bkeys_bits))
    pool = hier_pool(bs, n_entries, n_keep, block)
    valid = pool[pool >= 0]
    fine = indexer_scores(q_idx_bits, w, unpack_idx(idx_codes[valid],
                                                    idx_scales[valid]))
    sel = topk(fine, k, ids=valid)
    kv = gather_keys(main_codes, main_scales, sel, swa_codes, n_swa)
    return sel, mqa_decode(q_bits, kv, scale), pool, fine


def full_pool_layer(main_codes, main_scales, idx_codes, idx_scales,
                    n_entries, q_idx_bits, w, q_bits, swa_codes, n_swa, k,
                    scale, n_keep=2048, block=8):
    """First Full layer of a hierarchical decoder group, [KVC] 4.3 and
    [ARCH] 2.3.2 (Figure 5): the Full layer itself (its own top-k and
    attention over every visible entry), plus the candidate pool of the
    Reindex layers after it -- the n_keep blocks with the largest
    block_max_scores, expanded to their positions < n_entries, ascending.
    Returns (top-k ids, output, pool [n_keep * block], fine scores)."""
    sel, out, sc = full_layer(main_codes, main_scales, idx_codes, idx_scales,
                              n_entries, q_idx_bits, w, q_bits, swa_codes,
                              n_swa, k, scale)
    pool = hier_pool(block_max_scores(sc, n_entries, block), n_entries,
                     n_keep, block)
    return sel, out, pool, sc


def reindex_layer(main_codes, main_scales, idx_codes, idx_scales, pool,
                  q_idx_bits, w, q_bits, swa_codes, n_swa, k, scale):
    """Reindex-mode layer, [KVC] 4.2 table and 4.3 equation: the layer's own
    indexer query scores only the pool's positions (ids < 0 skipped) on the
    shared indexer keys, its top-k among them, then attention over the
    chosen main entries and the layer's own window.
    Returns (top-k ids, output, pool scores)."""
    pool = np.asarray(pool)
    valid = pool[pool >= 0]
    fine = indexer_scores(q_idx_bits, w, unpack_idx(idx_codes[valid],
                                                    idx_scales[valid]))
    sel = topk(fine, k, ids=valid)
    kv = gather_keys(main_codes, main_scales, sel, swa_codes, n_swa)
    return sel, mqa_decode(q_bits, kv, scale), fine


def reuse_layer_ext(main_codes, main_scales, sel, q_bits, swa_codes, n_swa,
                    scale, sink=None, pos=None, theta=10000.0):
    """Reuse-mode attention with the [V4] epilogue details: the per-head
    sink (mqa_decode_sink) and/or the partial-RoPE output de-rotation at the
    query position `pos` (rope_derotate)."""
    kv = gather_keys(main_codes, main_scales, sel, swa_codes, n_swa)
    o = (mqa_decode(q_bits, kv, scale) if sink is None
         else mqa_decode_sink(q_bits, kv, scale, sink))
    return o if pos is None else rope_derotate(o, pos, theta)


# ------------------------------------------------ write path (compressor) --
def softmax_pool(c, z):
    """Sequence compression of one block, [KVC] 4.1: the new entry is the
    per-channel softmax(Z)-weighted sum of the block's m token rows,
    C_bar = sum_i softmax_i(Z_i) (.) C_i.  c, z: float64 [m, 512]."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=0, keepdims=True))
    return (e * np.asarray(c, dtype=np.float64)).sum(axis=0) / e.sum(axis=0)


def compress_block(h_bits, w_kv_bits, w_z_bits, w_ik_bits):
    """The CSA2 write path for one block of m tokens, [KVC] 4.1 (main-KV,
    sequence-compression and indexer-K equations; [ARCH] 2.3): C = H W^KV
    and Z = H W^Z for the block's hidden states, C_bar = softmax_pool(C, Z)
    (non-overlapping blocks), and K^I = C_bar W^IK.  bf16 bits: h [m, d];
    w_kv, w_z [512, d] and w_ik [128, 512] (output x input).
    Returns (C [m, 512], C_bar [512], K^I [128]), float64."""
    h = F.bf16_bits_to_f64(h_bits)
    c = h @ F.bf16_bits_to_f64(w_kv_bits).T
    z = h @ F.bf16_bits_to_f64(w_z_bits).T
    cbar = softmax_pool(c, z)
    ki = cbar @ F.bf16_bits_to_f64(w_ik_bits).T
    return c, cbar, ki
