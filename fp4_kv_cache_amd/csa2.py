"""Python binding of libcsa2 (ctypes).  Argument marshalling only: every
step of the decode path runs in the library's HIP kernels.  Tensors are
torch device tensors; calls are enqueued on torch's current stream.

The names mirror the C ABI in include/csa2.h (csa2_pack_kv -> pack_kv, ...).
A missing or unloadable library raises immediately: there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

FMT_MAIN, FMT_IDX, FMT_SWA = 0, 1, 2
KEYS_MXFP4, KEYS_BF16 = 0, 1
OP_TOPK, OP_DECODE, OP_REUSE, OP_FULL_POOL, OP_REINDEX, OP_COMPRESS = (
    0, 1, 2, 3, 4, 5)
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "ALIGNMENT",
          4: "WORKSPACE", 5: "HIP"}
EXPORTS = ["csa2_pack_kv", "csa2_unpack_kv", "csa2_build_block_keys",
           "csa2_indexer_score", "csa2_indexer_score_fp4q", "csa2_topk",
           "csa2_sparse_attn_decode", "csa2_sparse_attn_decode_fp4q",
           "csa2_full_pool_decode", "csa2_reindex_decode", "csa2_reuse_attn",
           "csa2_sparse_attn_decode_ex", "csa2_reuse_attn_ex",
           "csa2_sparse_attn_decode_noalloc",
           "csa2_sparse_attn_decode_fp4q_ex", "csa2_full_pool_decode_ex",
           "csa2_reindex_decode_ex",
           "csa2_compress_append", "csa2_workspace_size", "csa2_entry_bytes",
           "csa2_kv_bytes_per_token", "csa2_set_launch_events",
           "csa2_launch_events_recorded",
           "csa2_last_error", "csa2_version"]


class Csa2Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libcsa2 {STATUS.get(status, status)}: {message}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("main_codes", ctypes.c_void_p),
                ("main_scales", ctypes.c_void_p),
                ("idx_codes", ctypes.c_void_p),
                ("idx_scales", ctypes.c_void_p),
                ("block_keys", ctypes.c_void_p),
                ("n_cap", ctypes.c_int64),
                ("n_entries", ctypes.c_void_p)]


class PoolOpts(ctypes.Structure):
    _fields_ = [("n_blocks_keep", ctypes.c_int32), ("block", ctypes.c_int32)]


class AttnOpts(ctypes.Structure):
    _fields_ = [("sink", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("rope_theta", ctypes.c_float)]


def _attn_opts(sink, pos, rope_theta):
    """csa2_attn_opts for the optional sink [64] float32 / positions [B]
    int32, or None when neither is given."""
    if sink is None and pos is None:
        return None
    if sink is not None:
        _need(sink, torch.float32, (64,), "sink")
    if pos is not None:
        _need(pos, torch.int32, name="pos")
    return AttnOpts(None if sink is None else sink.data_ptr(),
                    None if pos is None else pos.data_ptr(), float(rope_theta))


_lib = None

P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                        ctypes.c_float, ctypes.c_size_t)


def load(path=None):
    """Load libcsa2.so (built by `python -m fp4_kv_cache_amd.build`)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libcsa2 is not built: {p} is missing "
                          "(run python -m fp4_kv_cache_amd.build)")
    lib = ctypes.CDLL(p)
    sig = {
        "csa2_pack_kv": (I32, [I32, P, I64, P, P, P]),
        "csa2_unpack_kv": (I32, [I32, P, P, I64, P, P]),
        "csa2_build_block_keys": (I32, [P, P, I64, P, I32, I32, P, P]),
        "csa2_indexer_score": (I32, [I32, P, P, I64, P, P, I32, P, P, I32, P,
                                     P]),
        "csa2_indexer_score_fp4q": (I32, [I32, P, P, I64, P, P, I32, P, P,
                                          P, I32, P, P]),
        "csa2_topk": (I32, [P, I64, P, P, I32, I32, I32, P, P, P, SZ, P]),
        "csa2_sparse_attn_decode": (I32, [ctypes.POINTER(CacheDesc), P, P, P,
                                          P, P, I32, I32, F32,
                                          ctypes.POINTER(PoolOpts), P, P, P,
                                          SZ, P]),
        "csa2_sparse_attn_decode_fp4q": (I32, [ctypes.POINTER(CacheDesc), P,
                                               P, P, P, P, P, I32, I32, F32,
                                               ctypes.POINTER(PoolOpts), P, P,
                                               P, SZ, P]),
        "csa2_full_pool_decode": (I32, [ctypes.POINTER(CacheDesc), P, P, P,
                                        P, P, I32, I32, F32,
                                        ctypes.POINTER(PoolOpts), P, P, P, P,
                                        SZ, P]),
        "csa2_reindex_decode": (I32, [ctypes.POINTER(CacheDesc), P, I64, P,
                                      P, P, P, P, I32, I32, F32, P, P, P, SZ,
                                      P]),
        "csa2_sparse_attn_decode_fp4q_ex": (I32, [ctypes.POINTER(CacheDesc),
                                                  P, P, P, P, P, P, I32, I32,
                                                  F32, ctypes.POINTER(PoolOpts),
                                                  ctypes.POINTER(AttnOpts), P,
                                                  P, P, SZ, P]),
        "csa2_full_pool_decode_ex": (I32, [ctypes.POINTER(CacheDesc), P, P, P,
                                           P, P, I32, I32, F32,
                                           ctypes.POINTER(PoolOpts),
                                           ctypes.POINTER(AttnOpts), P, P, P,
                                           P, SZ, P]),
        "csa2_reindex_decode_ex": (I32, [ctypes.POINTER(CacheDesc), P, I64, P,
                                         P, P, P, P, I32, I32, F32,
                                         ctypes.POINTER(AttnOpts), P, P, P,
                                         SZ, P]),
        "csa2_sparse_attn_decode_ex": (I32, [ctypes.POINTER(CacheDesc), P, P,
                                             P, P, P, I32, I32, F32,
                                             ctypes.POINTER(PoolOpts),
                                             ctypes.POINTER(AttnOpts), P, P,
                                             P, SZ, P]),
        "csa2_sparse_attn_decode_noalloc": (I32, [ctypes.POINTER(CacheDesc),
                                                  P, P, P, P, P, I32, I32,
                                                  F32,
                                                  ctypes.POINTER(PoolOpts), P,
                                                  P, P]),
        "csa2_reuse_attn_ex": (I32, [P, P, I64, P, I32, P, P, P, I32, F32,
                                     ctypes.POINTER(AttnOpts), P, P, SZ, P]),
        "csa2_compress_append": (I32, [P, I32, I32, I32, P, P, P, P, P, P, P,
                                       P, I64, P, P, P, P, P, P, SZ, P]),
        "csa2_reuse_attn": (I32, [P, P, I64, P, I32, P, P, P, I32, F32, P, P,
                                  SZ, P]),
        "csa2_workspace_size": (SZ, [I32, I32, I64, I32,
                                     ctypes.POINTER(PoolOpts)]),
        "csa2_entry_bytes": (I32, [I32]),
        "csa2_kv_bytes_per_token": (ctypes.c_double,
                                    [ctypes.POINTER(I32), I32]),
        "csa2_set_launch_events": (I32, [ctypes.POINTER(ctypes.c_void_p),
                                         I32]),
        "csa2_launch_events_recorded": (I32, []),
        "csa2_last_error": (ctypes.c_char_p, []),
        "csa2_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def set_launch_events(events):
    """Benchmark hook: the next calls of the decode and reuse entry points
    record these HIP events (hipEvent_t handles as ctypes.c_void_p or int)
    before their first kernel and after each kernel; pass [] to clear."""
    arr = (ctypes.c_void_p * max(1, len(events)))(
        *[e if isinstance(e, ctypes.c_void_p) else ctypes.c_void_p(e)
          for e in events])
    _check(load().csa2_set_launch_events(arr, len(events)))


def launch_events_recorded():
    """Events recorded by the latest call made under set_launch_events."""
    return load().csa2_launch_events_recorded()


def _check(status):
    if status != 0:
        raise Csa2Error(status, load().csa2_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape=None, name="tensor"):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")


def version():
    return load().csa2_version().decode()


def entry_bytes(fmt):
    return load().csa2_entry_bytes(fmt)


def kv_bytes_per_token(m_of_kv_layers):
    arr = (I32 * len(m_of_kv_layers))(*m_of_kv_layers)
    return load().csa2_kv_bytes_per_token(arr, len(m_of_kv_layers))


def workspace_size(op, B, n_cap, k, pool=None):
    po = PoolOpts(*pool) if pool is not None else None
    return load().csa2_workspace_size(op, B, n_cap, k,
                                      ctypes.byref(po) if po else None)


def workspace(nbytes, device):
    """A 256-byte aligned device workspace of at least nbytes."""
    t = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8,
                    device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + max(int(nbytes), 1)]


# ------------------------------------------------------------------ calls --
def pack_kv(fmt, src, codes=None, scales=None):
    """Quantise float32 rows [n, 512|128] into (codes, scales)."""
    _need(src, torch.float32, name="src")
    n = src.shape[0]
    cw, sw = {FMT_MAIN: (256, 32), FMT_IDX: (64, 4), FMT_SWA: (512, 0)}[fmt]
    if codes is None:
        codes = torch.empty((n, cw), dtype=torch.uint8, device=src.device)
    if scales is None and sw:
        scales = torch.empty((n, sw), dtype=torch.uint8, device=src.device)
    _check(load().csa2_pack_kv(fmt, _ptr(src), n, _ptr(codes), _ptr(scales),
                               _stream()))
    return codes, scales


def unpack_kv(fmt, codes, scales=None):
    n = codes.shape[0]
    dim = 128 if fmt == FMT_IDX else 512
    out = torch.empty((n, dim), dtype=torch.float32, device=codes.device)
    _check(load().csa2_unpack_kv(fmt, _ptr(codes), _ptr(scales), n, _ptr(out),
                                 _stream()))
    return out


def build_block_keys(idx_codes, idx_scales, n_entries, block=8):
    """idx planes [B, n_cap, 64] / [B, n_cap, 4] -> bf16 keys [B, nb, 128]."""
    B, n_cap = idx_codes.shape[0], idx_codes.shape[1]
    nb = (n_cap + block - 1) // block
    out = torch.empty((B, nb, 128), dtype=torch.bfloat16,
                      device=idx_codes.device)
    _check(load().csa2_build_block_keys(_ptr(idx_codes), _ptr(idx_scales),
                                        n_cap, _ptr(n_entries), B, block,
                                        _ptr(out), _stream()))
    return out


def indexer_score(keyfmt, k_codes, k_scales, n_entries, q_idx, w, cand=None,
                  out=None):
    """Scores [B, n_cap] (or [B, n_cand] for candidate ids)."""
    B, n_cap = k_codes.shape[0], k_codes.shape[1]
    rows = n_cap if cand is None else cand.shape[1]
    if out is None:
        out = torch.empty((B, rows), dtype=torch.float32,
                          device=k_codes.device)
    _need(out, torch.float32, (B, rows), "out")
    _check(load().csa2_indexer_score(
        keyfmt, _ptr(k_codes), _ptr(k_scales), n_cap, _ptr(n_entries),
        _ptr(cand), 0 if cand is None else cand.shape[1], _ptr(q_idx),
        _ptr(w), B, _ptr(out), _stream()))
    return out


def pack_query_fp4(q_idx):
    """The MXFP4 planes of bf16 indexer queries [B, 32, 128]: codes
    [B, 32, 64] u8 and scales [B, 32, 4] u8 (csa2_pack_kv, FMT_IDX)."""
    B = q_idx.shape[0]
    codes, scales = pack_kv(FMT_IDX, q_idx.reshape(B * 32, 128).float())
    return codes.view(B, 32, 64), scales.view(B, 32, 4)


def indexer_score_fp4q(keyfmt, k_codes, k_scales, n_entries, q_codes,
                       q_scales, w, cand=None, out=None):
    """indexer_score with an MXFP4 query (pack_query_fp4 planes)."""
    B, n_cap = k_codes.shape[0], k_codes.shape[1]
    rows = n_cap if cand is None else cand.shape[1]
    if out is None:
        out = torch.empty((B, rows), dtype=torch.float32,
                          device=k_codes.device)
    _need(out, torch.float32, (B, rows), "out")
    _need(q_codes, torch.uint8, (B, 32, 64), "q_codes")
    _need(q_scales, torch.uint8, (B, 32, 4), "q_scales")
    _check(load().csa2_indexer_score_fp4q(
        keyfmt, _ptr(k_codes), _ptr(k_scales), n_cap, _ptr(n_entries),
        _ptr(cand), 0 if cand is None else cand.shape[1], _ptr(q_codes),
        _ptr(q_scales), _ptr(w), B, _ptr(out), _stream()))
    return out


def topk(scores, k, n_valid=None, ids=None, block=1, limit=None, ws=None,
         out=None):
    B, ld = scores.shape
    if out is None:
        out = torch.empty((B, k * block), dtype=torch.int32,
                          device=scores.device)
    _need(out, torch.int32, (B, k * block), "out")
    need = workspace_size(OP_TOPK, B, ld, k)
    if ws is None:
        ws = workspace(need, scores.device)
    _check(load().csa2_topk(_ptr(scores), ld, _ptr(n_valid), _ptr(ids), B, k,
                            block, _ptr(limit), _ptr(out), _ptr(ws),
                            ws.numel(), _stream()))
    return out


def cache_desc(main_codes, main_scales, idx_codes, idx_scales, n_entries,
               block_keys=None):
    return CacheDesc(main_codes.data_ptr(), main_scales.data_ptr(),
                     idx_codes.data_ptr(), idx_scales.data_ptr(),
                     0 if block_keys is None else block_keys.data_ptr(),
                     main_codes.shape[1], n_entries.data_ptr())


def sparse_attn_decode(cache, q_idx, w, q, swa, n_swa, k, scale, pool=None,
                       out=None, topk_out=None, ws=None, sink=None, pos=None,
                       rope_theta=10000.0):
    """One Full-layer decode step.  `cache` is a CacheDesc (keep the
    tensors it points to alive).  Returns (out bf16 [B,64,512], topk
    [B,k])."""
    B = q.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=dev)
    if topk_out is None:
        topk_out = torch.empty((B, k), dtype=torch.int32, device=dev)
    po = PoolOpts(*pool) if pool is not None else None
    if ws is None:
        need = load().csa2_workspace_size(OP_DECODE, B, cache.n_cap, k,
                                          ctypes.byref(po) if po else None)
        ws = workspace(need, dev)
    ao = _attn_opts(sink, pos, rope_theta)
    if ao is None:
        _check(load().csa2_sparse_attn_decode(
            ctypes.byref(cache), _ptr(q_idx), _ptr(w), _ptr(q), _ptr(swa),
            _ptr(n_swa), B, k, float(scale), ctypes.byref(po) if po else None,
            _ptr(out), _ptr(topk_out), _ptr(ws), ws.numel(), _stream()))
    else:
        _check(load().csa2_sparse_attn_decode_ex(
            ctypes.byref(cache), _ptr(q_idx), _ptr(w), _ptr(q), _ptr(swa),
            _ptr(n_swa), B, k, float(scale), ctypes.byref(po) if po else None,
            ctypes.byref(ao), _ptr(out), _ptr(topk_out), _ptr(ws), ws.numel(),
            _stream()))
    return out, topk_out


def sparse_attn_decode_noalloc(cache, q_idx, w, q, swa, n_swa, k, scale,
                               pool=None, out=None, topk_out=None):
    """sparse_attn_decode without a workspace: the library's own fixed
    scratch array (csa2_sparse_attn_decode_noalloc).  The outputs must be
    given by callers that cannot allocate."""
    B = q.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=dev)
    if topk_out is None:
        topk_out = torch.empty((B, k), dtype=torch.int32, device=dev)
    po = PoolOpts(*pool) if pool is not None else None
    _check(load().csa2_sparse_attn_decode_noalloc(
        ctypes.byref(cache), _ptr(q_idx), _ptr(w), _ptr(q), _ptr(swa),
        _ptr(n_swa), B, k, float(scale), ctypes.byref(po) if po else None,
        _ptr(out), _ptr(topk_out), _stream()))
    return out, topk_out


def sparse_attn_decode_fp4q(cache, q_codes, q_scales, w, q, swa, n_swa, k,
                            scale, pool=None, out=None, topk_out=None,
                            ws=None, sink=None, pos=None, rope_theta=10000.0):
    """sparse_attn_decode with an MXFP4 indexer query (pack_query_fp4
    planes)."""
    B = q.shape[0]
    dev = q.device
    _need(q_codes, torch.uint8, (B, 32, 64), "q_codes")
    _need(q_scales, torch.uint8, (B, 32, 4), "q_scales")
    if out is None:
        out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=dev)
    if topk_out is None:
        topk_out = torch.empty((B, k), dtype=torch.int32, device=dev)
    po = PoolOpts(*pool) if pool is not None else None
    if ws is None:
        need = load().csa2_workspace_size(OP_DECODE, B, cache.n_cap, k,
                                          ctypes.byref(po) if po else None)
        ws = workspace(need, dev)
    ao = _attn_opts(sink, pos, rope_theta)
    if ao is None:
        _check(load().csa2_sparse_attn_decode_fp4q(
            ctypes.byref(cache), _ptr(q_codes), _ptr(q_scales), _ptr(w),
            _ptr(q), _ptr(swa), _ptr(n_swa), B, k, float(scale),
            ctypes.byref(po) if po else None, _ptr(out), _ptr(topk_out),
            _ptr(ws), ws.numel(), _stream()))
    else:
        _check(load().csa2_sparse_attn_decode_fp4q_ex(
            ctypes.byref(cache), _ptr(q_codes), _ptr(q_scales), _ptr(w),
            _ptr(q), _ptr(swa), _ptr(n_swa), B, k, float(scale),
            ctypes.byref(po) if po else None, ctypes.byref(ao), _ptr(out),
            _ptr(topk_out), _ptr(ws), ws.numel(), _stream()))
    return out, topk_out


def full_pool_decode(cache, q_idx, w, q, swa, n_swa, k, scale,
                     pool=(2048, 8), out=None, topk_out=None, pool_out=None,
                     ws=None, sink=None, pos=None, rope_theta=10000.0):
    """First Full layer of a hierarchical decoder group: returns (out bf16
    [B,64,512], topk [B,k], pool [B, n_blocks_keep*8])."""
    B = q.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=dev)
    if topk_out is None:
        topk_out = torch.empty((B, k), dtype=torch.int32, device=dev)
    if pool_out is None:
        pool_out = torch.empty((B, pool[0] * pool[1]), dtype=torch.int32,
                               device=dev)
    po = PoolOpts(*pool)
    if ws is None:
        need = load().csa2_workspace_size(OP_FULL_POOL, B, cache.n_cap, k,
                                          ctypes.byref(po))
        ws = workspace(need, dev)
    ao = _attn_opts(sink, pos, rope_theta)
    if ao is None:
        _check(load().csa2_full_pool_decode(
            ctypes.byref(cache), _ptr(q_idx), _ptr(w), _ptr(q), _ptr(swa),
            _ptr(n_swa), B, k, float(scale), ctypes.byref(po), _ptr(out),
            _ptr(topk_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream()))
    else:
        _check(load().csa2_full_pool_decode_ex(
            ctypes.byref(cache), _ptr(q_idx), _ptr(w), _ptr(q), _ptr(swa),
            _ptr(n_swa), B, k, float(scale), ctypes.byref(po),
            ctypes.byref(ao), _ptr(out), _ptr(topk_out), _ptr(pool_out),
            _ptr(ws), ws.numel(), _stream()))
    return out, topk_out, pool_out


def reindex_decode(cache, pool_ids, q_idx, w, q, swa, n_swa, k, scale,
                   out=None, topk_out=None, ws=None, sink=None, pos=None,
                   rope_theta=10000.0):
    """Reindex layer over a pool [B, n_pool]: returns (out, topk)."""
    B, n_pool = pool_ids.shape
    dev = q.device
    _need(pool_ids, torch.int32, name="pool_ids")
    if out is None:
        out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=dev)
    if topk_out is None:
        topk_out = torch.empty((B, k), dtype=torch.int32, device=dev)
    if ws is None:
        need = load().csa2_workspace_size(OP_REINDEX, B, n_pool, k, None)
        ws = workspace(need, dev)
    ao = _attn_opts(sink, pos, rope_theta)
    if ao is None:
        _check(load().csa2_reindex_decode(
            ctypes.byref(cache), _ptr(pool_ids), n_pool, _ptr(q_idx), _ptr(w),
            _ptr(q), _ptr(swa), _ptr(n_swa), B, k, float(scale), _ptr(out),
            _ptr(topk_out), _ptr(ws), ws.numel(), _stream()))
    else:
        _check(load().csa2_reindex_decode_ex(
            ctypes.byref(cache), _ptr(pool_ids), n_pool, _ptr(q_idx), _ptr(w),
            _ptr(q), _ptr(swa), _ptr(n_swa), B, k, float(scale),
            ctypes.byref(ao), _ptr(out), _ptr(topk_out), _ptr(ws), ws.numel(),
            _stream()))
    return out, topk_out


def reuse_attn(main_codes, main_scales, topk_ids, q, swa, n_swa, scale,
               out=None, ws=None, sink=None, pos=None, rope_theta=10000.0):
    B, k = topk_ids.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(workspace_size(OP_REUSE, B, main_codes.shape[1], k), dev)
    ao = _attn_opts(sink, pos, rope_theta)
    if ao is None:
        _check(load().csa2_reuse_attn(
            _ptr(main_codes), _ptr(main_scales), main_codes.shape[1],
            _ptr(topk_ids), k, _ptr(q), _ptr(swa), _ptr(n_swa), B,
            float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    else:
        _check(load().csa2_reuse_attn_ex(
            _ptr(main_codes), _ptr(main_scales), main_codes.shape[1],
            _ptr(topk_ids), k, _ptr(q), _ptr(swa), _ptr(n_swa), B,
            float(scale), ctypes.byref(ao), _ptr(out), _ptr(ws), ws.numel(),
            _stream()))
    return out


def compress_append(h, w_kv, w_z, w_ik, rows, main_codes, main_scales,
                    idx_codes, idx_scales, swa=None, swa_slot=None,
                    debug=False, ws=None):
    """The decode-time write path: h [B, m, d] bf16 -> one new entry per
    sequence at rows [B] (int32) of the caches ([B, n_cap, ...]); the m
    rows C_i go to window slots (swa_slot + i) mod 128 when swa is given.
    With debug=True returns (C_bar [B,512], K^I [B,128], C [B,m,512])
    float32."""
    B, m, d = h.shape
    _need(h, torch.bfloat16, name="h")
    for t, shp, nm in ((w_kv, (512, d), "w_kv"), (w_z, (512, d), "w_z"),
                       (w_ik, (128, 512), "w_ik")):
        _need(t, torch.bfloat16, shp, nm)
    _need(rows, torch.int32, (B,), "rows")
    dev = h.device
    outs = (None, None, None)
    if debug:
        outs = (torch.empty((B, 512), dtype=torch.float32, device=dev),
                torch.empty((B, 128), dtype=torch.float32, device=dev),
                torch.empty((B, m, 512), dtype=torch.float32, device=dev))
    if ws is None:
        ws = workspace(load().csa2_workspace_size(OP_COMPRESS, B, m, d, None),
                       dev)
    _check(load().csa2_compress_append(
        _ptr(h), B, m, d, _ptr(w_kv), _ptr(w_z), _ptr(w_ik), _ptr(rows),
        _ptr(main_codes), _ptr(main_scales), _ptr(idx_codes),
        _ptr(idx_scales), main_codes.shape[1], _ptr(swa), _ptr(swa_slot),
        _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(ws), ws.numel(),
        _stream()))
    return outs if debug else None
