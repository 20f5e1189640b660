"""Device-resident caches and queries of a synthetic CSA2 workload, built
with the library's own packing kernels (the write path).

    st = build(WORKLOADS[1], device="cuda")
    out, ids = csa2.sparse_attn_decode(st.cache, st.q_idx, st.w, st.q[0],
                                       st.swa[0], st.n_swa, 512, st.scale)
"""
import math
from dataclasses import dataclass

import torch

from . import csa2, inputs
from .inputs import CHUNK


@dataclass
class DeviceWorkload:
    wl: inputs.Workload
    main_codes: torch.Tensor      # [B, n, 256] u8
    main_scales: torch.Tensor     # [B, n, 32] u8
    idx_codes: torch.Tensor       # [B, n, 64] u8
    idx_scales: torch.Tensor      # [B, n, 4] u8
    block_keys: torch.Tensor      # [B, nb, 128] bf16 or None
    n_entries: torch.Tensor       # [B] i32
    q_idx: torch.Tensor           # [B, 32, 128] bf16
    w: torch.Tensor               # [B, 32] f32
    q: list                       # per layer [B, 64, 512] bf16
    swa: list                     # per layer [B, 128, 512] u8
    n_swa: torch.Tensor           # [B] i32
    scale: float
    cache: csa2.CacheDesc = None

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   [self.main_codes, self.main_scales, self.idx_codes,
                    self.idx_scales] + ([self.block_keys]
                                        if self.block_keys is not None else []))


def attn_scale():
    """1/sqrt(c) with c = 512, as float32."""
    return float(torch.tensor(1.0 / math.sqrt(512.0), dtype=torch.float32))


def build(wl, device="cuda", seqs=None):
    """Generate and pack every cache of workload `wl` on `device`.

    seqs: optional list of sequence ids to materialise (others stay zero)."""
    B, n = wl.B, wl.n
    dev = torch.device(device)
    mc = torch.empty((B, n, 256), dtype=torch.uint8, device=dev)
    ms = torch.empty((B, n, 32), dtype=torch.uint8, device=dev)
    ic = torch.empty((B, n, 64), dtype=torch.uint8, device=dev)
    isc = torch.empty((B, n, 4), dtype=torch.uint8, device=dev)
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        for c0 in range(0, n, CHUNK):
            c1 = min(n, c0 + CHUNK)
            x = inputs.main_latents(wl, b, c0, c1, dev)
            csa2.pack_kv(csa2.FMT_MAIN, x, mc[b, c0:c1], ms[b, c0:c1])
            y = inputs.idx_latents(wl, b, c0, c1, dev)
            csa2.pack_kv(csa2.FMT_IDX, y, ic[b, c0:c1], isc[b, c0:c1])
            del x, y
    n_entries = torch.full((B,), n, dtype=torch.int32, device=dev)
    bk = None
    if wl.pool is not None:
        bk = csa2.build_block_keys(ic, isc, n_entries, wl.pool[1])
    qi, ww = zip(*[inputs.index_query(wl, b, dev) for b in range(B)])
    layers = 1 + wl.reuse_layers
    q, swa = [], []
    for layer in range(layers):
        q.append(torch.stack([inputs.attn_query(wl, b, layer, dev)
                              for b in range(B)]))
        s = torch.empty((B, 128, 512), dtype=torch.uint8, device=dev)
        for b in range(B):
            csa2.pack_kv(csa2.FMT_SWA, inputs.window_latents(wl, b, layer, dev),
                         s[b])
        swa.append(s)
    st = DeviceWorkload(wl, mc, ms, ic, isc, bk, n_entries,
                        torch.stack(qi).contiguous(), torch.stack(ww).contiguous(),
                        q, swa, torch.full((B,), wl.n_swa, dtype=torch.int32,
                                           device=dev), attn_scale())
    st.cache = csa2.cache_desc(mc, ms, ic, isc, n_entries, bk)
    return st
