"""Decode steps captured in a HIP graph (the way the throughput is timed)
replay the eager results bit for bit.

The graph holds a Full-layer decode (bf16 indexer query), a Reuse layer on
its top-k ids, and a hierarchical-pool decode, each writing preallocated
outputs through caller workspaces.  It is replayed several times with
unrelated eager work and synchronisations between the replays, and every
replay is compared with the eager outputs (outputs cleared before each
replay, so a replay that skipped a kernel would show)."""
import dataclasses

import pytest
import torch

from fp4_kv_cache_amd import csa2, workload
from fp4_kv_cache_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_graph_replays_match_eager():
    wl = dataclasses.replace(WORKLOADS[1], cid=106, B=3, n=20000)
    st = workload.build(wl, DEV)
    wlp = dataclasses.replace(WORKLOADS[4], cid=107, B=2, n=8 * 4000 + 5,
                              pool=(256, 8))
    sp = workload.build(wlp, DEV)
    B, k = wl.B, wl.k
    assert wlp.k == k
    ws_d = csa2.workspace(csa2.workspace_size(csa2.OP_DECODE, B, wl.n, k), DEV)
    ws_r = csa2.workspace(csa2.workspace_size(csa2.OP_REUSE, B, wl.n, k), DEV)
    ws_p = csa2.workspace(csa2.workspace_size(csa2.OP_DECODE, wlp.B, wlp.n,
                                              k, wlp.pool), DEV)
    out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((B, k), dtype=torch.int32, device=DEV)
    out_r = torch.empty_like(out)
    out_p = torch.empty((wlp.B, 64, 512), dtype=torch.bfloat16, device=DEV)
    ids_p = torch.empty((wlp.B, k), dtype=torch.int32, device=DEV)
    outs = (out, ids, out_r, out_p, ids_p)

    def step():
        csa2.sparse_attn_decode(st.cache, st.q_idx, st.w, st.q[0], st.swa[0],
                                st.n_swa, k, st.scale, out=out, topk_out=ids,
                                ws=ws_d)
        csa2.reuse_attn(st.main_codes, st.main_scales, ids, st.q[1 % len(st.q)],
                        st.swa[1 % len(st.swa)], st.n_swa, st.scale,
                        out=out_r, ws=ws_r)
        csa2.sparse_attn_decode(sp.cache, sp.q_idx, sp.w, sp.q[0], sp.swa[0],
                                sp.n_swa, k, sp.scale, pool=wlp.pool,
                                out=out_p, topk_out=ids_p, ws=ws_p)

    step()
    torch.cuda.synchronize()
    eager = [_bits(t).clone() for t in outs]
    assert (eager[1] >= 0).any() and (eager[4] >= 0).any()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn((1 << 20,), device=DEV)
    for rep in range(4):
        for t in outs:
            _bits(t).fill_(-7)
        # unrelated eager work on the same device between replays
        other.mul_(1.5).add_(0.25)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("out", "ids", "reuse", "pool out", "pool ids"),
                              outs, eager):
            assert torch.equal(_bits(t), e), (rep, name)
    del g
