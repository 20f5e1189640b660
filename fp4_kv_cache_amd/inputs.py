"""Seeded synthetic inputs for the CSA2 decode workloads.

This module only draws numbers (it holds none of the method's arithmetic:
no quantisation, scoring or attention).  Both the GPU path and the CPU
oracle consume what it returns.  Every tensor is drawn with torch's
generator on the requested device from a seed derived with NumPy's
SeedSequence from (config, tensor, sequence, chunk), in chunks of 65,536
rows, so any row range can be regenerated on its own.  A given device
always yields the same values; CPU and GPU draws differ, so a test that
compares the two sides draws once and hands both the same tensor.

Workloads (value distributions as stated for each configuration):
  main-KV latents  N(0, 1) float32 [n, 512]   (packed E2M1 + E4M3 / 16)
  indexer keys     N(0, 1) float32 [n, 128]   (packed MXFP4), plus, in the
                   planted workload, +3 * v/|v| on a seeded 1 % of rows,
                   v = sum_h w_h q_h (a 3-sigma shift of the linear
                   similarity w . (q k) under k ~ N(0, I))
  indexer query    N(0, 1) rounded to bf16 [32, 128]; weights U(0, 1) [32]
  attention query  N(0, 1) rounded to bf16 [64, 512]
  window rows      N(0, 1) float32 [128, 512] (packed E4M3)
"""
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 65536
D_MAIN, D_IDX, H_IDX, H_ATTN, N_WIN = 512, 128, 32, 64, 128


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    B: int
    n: int                  # compressed entries per sequence
    ctx: int                # context tokens
    m: int                  # compression ratio
    k: int = 512
    n_swa: int = N_WIN
    reuse_layers: int = 0   # Reuse layers after the Full layer
    planted: float = 0.0    # fraction of planted indexer keys
    pool: tuple = None      # (blocks kept, block size) for the hierarchy
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    0: Workload(0, "tiny-2k", B=1, n=1024, ctx=2048, m=2),
    1: Workload(1, "encoder-full-64k", B=32, n=32768, ctx=65536, m=2),
    2: Workload(2, "decoder-group-128k", B=64, n=131072, ctx=131072, m=1,
                reuse_layers=3),
    3: Workload(3, "planted-1m", B=4, n=524288, ctx=1048576, m=2,
                planted=0.01),
    4: Workload(4, "hierarchical-1m", B=8, n=1048576, ctx=1048576, m=1,
                pool=(2048, 8)),
}

T_MAIN, T_IDX, T_QIDX, T_W, T_Q, T_SWA, T_PLANT = 1, 2, 3, 4, 5, 6, 7
T_HID, T_WKV, T_WZ, T_WIK = 8, 9, 10, 11


def seed(cid, tensor, seq, chunk=0, layer=0):
    ss = np.random.SeedSequence(0, spawn_key=(cid, tensor, layer, seq, chunk))
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, s):
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, s, device):
    return torch.randn(shape, generator=_gen(device, s), device=device,
                       dtype=torch.float32)


def main_latents(wl, b, lo, hi, device="cpu"):
    """Rows lo..hi-1 of sequence b's main-KV latents, float32 [hi-lo, 512]."""
    return _rows(wl, T_MAIN, D_MAIN, b, lo, hi, device)


def _rows(wl, tensor, dim, b, lo, hi, device):
    parts = []
    for c in range(lo // CHUNK, (hi + CHUNK - 1) // CHUNK):
        c0 = c * CHUNK
        rows = min(CHUNK, wl.n - c0)
        x = _normal((rows, dim), seed(wl.cid, tensor, b, c), device)
        a, z = max(lo, c0) - c0, min(hi, c0 + rows) - c0
        parts.append(x[a:z])
    if not parts:
        return torch.empty((0, dim), dtype=torch.float32, device=device)
    return torch.cat(parts) if len(parts) > 1 else parts[0]


def index_query(wl, b, device="cpu", layer=0):
    """(q_idx bf16 [32, 128], w float32 [32]) of sequence b in a layer (a
    Reindex layer has its own indexer query)."""
    q = _normal((H_IDX, D_IDX), seed(wl.cid, T_QIDX, b, layer=layer), device)
    w = torch.rand((H_IDX,), generator=_gen(device, seed(wl.cid, T_W, b,
                                                         layer=layer)),
                   device=device, dtype=torch.float32)
    return q.to(torch.bfloat16), w


def planted_rows(wl, b, device="cpu"):
    """Sorted ids of the planted indexer keys of sequence b (may be empty)."""
    cnt = int(np.floor(wl.planted * wl.n))
    if cnt == 0:
        return torch.empty(0, dtype=torch.int64, device=device)
    perm = torch.randperm(wl.n, generator=_gen(device, seed(wl.cid, T_PLANT, b)),
                          device=device)
    return torch.sort(perm[:cnt]).values


def idx_latents(wl, b, lo, hi, device="cpu"):
    """Rows lo..hi-1 of sequence b's indexer keys, float32 [hi-lo, 128]."""
    x = _rows(wl, T_IDX, D_IDX, b, lo, hi, device)
    if wl.planted > 0:
        q, w = index_query(wl, b, device)
        v = (w[:, None] * q.float()).sum(0)
        u = v / torch.linalg.vector_norm(v)
        pr = planted_rows(wl, b, device)
        sel = pr[(pr >= lo) & (pr < hi)] - lo
        x[sel] += 3.0 * u
    return x


def attn_query(wl, b, layer=0, device="cpu"):
    """bf16 [64, 512] attention query of sequence b in a layer."""
    return _normal((H_ATTN, D_MAIN), seed(wl.cid, T_Q, b, layer=layer),
                   device).to(torch.bfloat16)


def window_latents(wl, b, layer=0, device="cpu"):
    """float32 [128, 512] window rows of sequence b in a layer."""
    return _normal((N_WIN, D_MAIN), seed(wl.cid, T_SWA, b, layer=layer),
                   device)


def hidden_states(cid, B, m, d, device="cpu"):
    """bf16 [B, m, d] hidden states (N(0,1)) of the m newest tokens."""
    return _normal((B, m, d), seed(cid, T_HID, 0), device).to(torch.bfloat16)


def compressor_weights(cid, d, device="cpu"):
    """Synthetic write-path weights, bf16, [out][in]: W^KV and W^Z [512, d]
    and W^IK [128, 512], N(0, 1/in) so that the projections of N(0,1)
    inputs have unit variance."""
    wkv = _normal((512, d), seed(cid, T_WKV, 0), device) / d ** 0.5
    wz = _normal((512, d), seed(cid, T_WZ, 0), device) / d ** 0.5
    wik = _normal((128, 512), seed(cid, T_WIK, 0), device) / 512 ** 0.5
    return (wkv.to(torch.bfloat16), wz.to(torch.bfloat16),
            wik.to(torch.bfloat16))
