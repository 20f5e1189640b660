"""The attention details of the V4 page on the GPU against the oracle: the
per-head sink logit in the softmax denominator and the partial-RoPE output
de-rotation by the query position.  Both places that finish an output are
covered: the attention kernel itself (one split per sequence, many
sequences) and the split merge (few sequences, several splits)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2, inputs, workload
from fp4_kv_cache_amd.inputs import WORKLOADS
from _util import REL_L2_TOL, bf16_bits, rel_l2, topk_set_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = float(np.float32(1.0 / math.sqrt(512)))


def _cache(B, n, seed):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((B * n, 512)).astype(np.float32)).to(DEV)
    mc, ms = csa2.pack_kv(csa2.FMT_MAIN, x)
    sw = torch.from_numpy(rng.standard_normal((B * 128, 512)).astype(np.float32)).to(DEV)
    swc, _ = csa2.pack_kv(csa2.FMT_SWA, sw)
    q = torch.from_numpy(rng.standard_normal((B, 64, 512)).astype(np.float32))
    return (mc.view(B, n, 256), ms.view(B, n, 32), swc.view(B, 128, 512),
            q.to(torch.bfloat16).to(DEV))


def _ids(B, n, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([np.sort(rng.choice(n, size=k, replace=False))
                    for _ in range(B)]).astype(np.int32)
    ids[0, -3:] = -1                                 # a few empty slots
    return ids


@pytest.mark.parametrize("B,n,k,check", [(3, 900, 64, (0, 1, 2)),
                                         (3, 900, 7, (0, 2)),
                                         (260, 700, 512, (0, 129, 259))])
def test_reuse_sink_and_derotation(B, n, k, check):
    mc, ms, swc, q = _cache(B, n, 40 + B)
    ids = _ids(B, n, k, 41)
    rng = np.random.default_rng(42)
    sink = rng.normal(0, 2, 64).astype(np.float32)
    sink[:4] = [-np.inf, 8.0, -8.0, 0.0]
    pos = rng.integers(0, 1 << 24, B).astype(np.int32)
    pos[:2] = [0, (1 << 24) - 1]
    n_swa = torch.full((B,), 128, dtype=torch.int32, device=DEV)
    n_swa[1] = 5
    tid = torch.from_numpy(ids).to(DEV)
    s_t = torch.from_numpy(sink).to(DEV)
    p_t = torch.from_numpy(pos).to(DEV)
    out = {}
    for name, kw in {"sink": dict(sink=s_t), "rope": dict(pos=p_t),
                     "both": dict(sink=s_t, pos=p_t, rope_theta=50000.0)}.items():
        out[name] = csa2.reuse_attn(mc, ms, tid, q, swc, n_swa, SCALE,
                                    **kw).float().cpu().numpy()
    plain = csa2.reuse_attn(mc, ms, tid, q, swc, n_swa, SCALE).float().cpu().numpy()
    mcc, msc, swh = mc.cpu().numpy(), ms.cpu().numpy(), swc.cpu().numpy()
    ns = n_swa.cpu().numpy()
    for b in check:
        qb = bf16_bits(q[b])
        args = (mcc[b], msc[b], ids[b], qb, swh[b], int(ns[b]), SCALE)
        refs = {"sink": O.reuse_layer_ext(*args, sink=sink),
                "rope": O.reuse_layer_ext(*args, pos=int(pos[b])),
                "both": O.reuse_layer_ext(*args, sink=sink, pos=int(pos[b]),
                                          theta=50000.0)}
        for name, ref in refs.items():
            e = rel_l2(out[name][b], ref)
            assert e <= REL_L2_TOL, (b, name, e)
        # options off: the plain call, unchanged
        assert rel_l2(plain[b], O.reuse_layer(*args)) <= REL_L2_TOL
        print(B, k, b, "ok", flush=True)


def test_decode_ex_sink_and_derotation():
    wl = dataclasses.replace(WORKLOADS[1], cid=401, B=3, n=6000)
    st = workload.build(wl, DEV)
    rng = np.random.default_rng(43)
    sink = torch.from_numpy(rng.normal(0, 1, 64).astype(np.float32)).to(DEV)
    pos = torch.tensor([123, 999999, 2 * 6000 + 1], dtype=torch.int32,
                       device=DEV)
    out, ids = csa2.sparse_attn_decode(st.cache, st.q_idx, st.w, st.q[0],
                                       st.swa[0], st.n_swa, wl.k, st.scale,
                                       sink=sink, pos=pos)
    out, ids = out.float().cpu().numpy(), ids.cpu().numpy()
    for b in range(wl.B):
        y = inputs.idx_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
        ic, isc = O.pack_idx(y)
        qi, w = inputs.index_query(wl, b, DEV)
        sc = O.indexer_scores(bf16_bits(qi), w.cpu().numpy(),
                              O.unpack_idx(ic, isc))
        ok, msg = topk_set_ok(ids[b], sc, wl.k)
        assert ok, (b, msg)
        x = inputs.main_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
        mc, ms = O.pack_main(x)
        sw = O.pack_swa(inputs.window_latents(wl, b, 0, DEV).cpu().numpy())
        ref = O.reuse_layer_ext(mc, ms, ids[b], bf16_bits(st.q[0][b]), sw,
                                wl.n_swa, st.scale, sink=sink.cpu().numpy(),
                                pos=int(pos[b]))
        e = rel_l2(out[b], ref)
        assert e <= REL_L2_TOL, (b, e)
        print(b, msg, f"rel-L2 {e:.2e}", flush=True)


def test_group_and_fp4q_ex_sink_and_derotation():
    """The sink and de-rotation through the other layer calls: the decoder
    group's Full layer with its pool (csa2_full_pool_decode_ex), a Reindex
    layer on that pool (csa2_reindex_decode_ex) and the MXFP4-query decode
    (csa2_sparse_attn_decode_fp4q_ex); each output against the oracle's
    attention with the same details over the call's own ids."""
    wl = dataclasses.replace(WORKLOADS[2], cid=402, B=3, n=7000,
                             reuse_layers=1)
    st = workload.build(wl, DEV)
    rng = np.random.default_rng(47)
    sink = torch.from_numpy(rng.normal(0, 1, 64).astype(np.float32)).to(DEV)
    pos = torch.tensor([7, 654321, 3 * 7000 - 1], dtype=torch.int32,
                       device=DEV)
    out0, ids0, pool = csa2.full_pool_decode(
        st.cache, st.q_idx, st.w, st.q[0], st.swa[0], st.n_swa, wl.k,
        st.scale, pool=(64, 8), sink=sink, pos=pos)
    qi1, w1 = (torch.stack(t).contiguous() for t in zip(*[
        inputs.index_query(wl, b, DEV, layer=1) for b in range(wl.B)]))
    out1, ids1 = csa2.reindex_decode(st.cache, pool, qi1, w1, st.q[1],
                                     st.swa[1], st.n_swa, wl.k, st.scale,
                                     sink=sink, pos=pos)
    qc, qs = csa2.pack_query_fp4(st.q_idx)
    out2, ids2 = csa2.sparse_attn_decode_fp4q(
        st.cache, qc, qs, st.w, st.q[0], st.swa[0], st.n_swa, wl.k, st.scale,
        sink=sink, pos=pos)
    torch.cuda.synchronize()
    sk = sink.cpu().numpy()
    for b in range(wl.B):
        x = inputs.main_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
        mc, ms = O.pack_main(x)
        for name, o, i, layer in (("full_pool", out0, ids0, 0),
                                  ("reindex", out1, ids1, 1),
                                  ("fp4q", out2, ids2, 0)):
            sw = O.pack_swa(inputs.window_latents(wl, b, layer, DEV).cpu().numpy())
            ib = i[b].cpu().numpy()
            assert np.all(np.diff(ib[ib >= 0]) > 0), (name, b)
            ref = O.reuse_layer_ext(mc, ms, ib, bf16_bits(st.q[layer][b]), sw,
                                    wl.n_swa, st.scale, sink=sk,
                                    pos=int(pos[b]))
            e = rel_l2(o[b].float().cpu().numpy(), ref)
            assert e <= REL_L2_TOL, (name, b, e)
            print(name, b, f"rel-L2 {e:.2e}", flush=True)
