"""The pages' hierarchical decoder group on the GPU against the oracle: the
first Full layer (its own top-k and attention, plus the pool of the blocks
with the largest maximum fine score) and Reindex layers that score only the
pool with their own indexer query.

Top-k sets follow the gap rule (the pool by the gap of the block maxima at
the n_keep boundary), attention is compared at rel-L2 <= 5e-3 on the GPU's
own id set, and every Reindex layer is checked on the GPU's pool."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2, inputs, workload
from fp4_kv_cache_amd.inputs import WORKLOADS
from _util import GAP_TOL, REL_L2_TOL, bf16_bits, rel_l2, topk_set_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer_query(wl, B, layer):
    qi, w = zip(*[inputs.index_query(wl, b, DEV, layer=layer) for b in range(B)])
    return torch.stack(qi).contiguous(), torch.stack(w).contiguous()


def _attn_ok(wl, st, b, layer, ids_b, out_b):
    gv = ids_b[ids_b >= 0]
    sel = torch.from_numpy(gv.astype(np.int64)).to(DEV)
    x = inputs.main_latents(wl, b, 0, wl.n, DEV)[sel].cpu().numpy()
    mc, ms = O.pack_main(x)
    assert np.array_equal(st.main_codes[b][sel].cpu().numpy(), mc)
    sw = O.pack_swa(inputs.window_latents(wl, b, layer, DEV).cpu().numpy())
    keys = np.concatenate([O.unpack_main(mc, ms), O.unpack_swa(sw[:wl.n_swa])])
    ref = O.mqa_decode(bf16_bits(st.q[layer][b]), keys, st.scale)
    e = rel_l2(out_b, ref)
    assert e <= REL_L2_TOL, (b, layer, e)
    return e


def _check_group(wl, st, ne, n_keep, k, res):
    (out0, ids0, pool), reidx = res
    for b in range(wl.B):
        n = ne[b]
        y = inputs.idx_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
        ic, isc = O.pack_idx(y)
        qi, w = inputs.index_query(wl, b, DEV)
        sc = O.indexer_scores(bf16_bits(qi), w.cpu().numpy(),
                              O.unpack_idx(ic[:n], isc[:n]))
        ok, msg = topk_set_ok(ids0[b], sc, k)
        assert ok, (b, "full", msg)
        e = _attn_ok(wl, st, b, 0, ids0[b], out0[b])
        # the pool: the n_keep blocks with the largest maximum fine score
        bs = O.block_max_scores(sc, n, 8)
        kb = min(n_keep, len(bs))
        gp = pool[b]
        gv = gp[gp >= 0]
        assert np.all(np.diff(gv) > 0) and np.all(gv < n)
        if O.topk_gap(bs, kb) >= GAP_TOL or kb == len(bs):
            assert np.array_equal(gp, O.hier_pool(bs, n, n_keep, 8)), b
            pmsg = "pool equal"
        else:
            thr = np.sort(bs)[::-1][kb - 1]
            assert np.all(bs[np.unique(gv // 8)] >= thr * (1 - GAP_TOL)), b
            pmsg = "pool near-tie; membership checked"
        errs = [e]
        for layer, (out_l, ids_l) in reidx.items():
            qi_l, w_l = inputs.index_query(wl, b, DEV, layer=layer)
            fine = O.indexer_scores(bf16_bits(qi_l), w_l.cpu().numpy(),
                                    O.unpack_idx(ic[gv], isc[gv]))
            ok, msg_l = topk_set_ok(ids_l[b], fine, k, ids=gv)
            assert ok, (b, layer, msg_l)
            errs.append(_attn_ok(wl, st, b, layer, ids_l[b], out_l[b]))
        print(b, f"n={n}", msg, pmsg, "rel-L2", [f"{x:.2e}" for x in errs],
              flush=True)


def _run(wl, st, n_keep, k, layers):
    out0, ids0, pool = csa2.full_pool_decode(st.cache, st.q_idx, st.w, st.q[0],
                                             st.swa[0], st.n_swa, k, st.scale,
                                             pool=(n_keep, 8))
    reidx = {}
    for layer in layers:
        qi_l, w_l = _layer_query(wl, wl.B, layer)
        reidx[layer] = csa2.reindex_decode(st.cache, pool, qi_l, w_l,
                                           st.q[layer], st.swa[layer],
                                           st.n_swa, k, st.scale)
    torch.cuda.synchronize()
    return ((out0.float().cpu().numpy(), ids0.cpu().numpy(),
             pool.cpu().numpy()),
            {l: (o.float().cpu().numpy(), i.cpu().numpy())
             for l, (o, i) in reidx.items()})


@pytest.mark.parametrize("n_keep", [64, 2048])
def test_group_small_ragged(n_keep):
    """n_keep = 64: the block top-k takes the tile-pruned path; 2048: the
    streaming path, and sequence 2's 100 blocks are all kept."""
    wl = dataclasses.replace(WORKLOADS[2], cid=302, B=3, n=20003,
                             reuse_layers=2)
    st = workload.build(wl, DEV)
    ne = [20003, 9001, 800]
    st.n_entries.copy_(torch.tensor(ne, dtype=torch.int32))
    k = 256 if n_keep == 64 else 512
    _check_group(wl, st, ne, n_keep, k, _run(wl, st, n_keep, k, (1, 2)))


def test_group_full_size_sampled():
    """The decoder-group shapes (64 sequences x 131,072 entries) with the
    pages' pool (2,048 blocks of 8) and one Reindex layer; sequences 0 and
    63 checked."""
    wl = dataclasses.replace(WORKLOADS[2], reuse_layers=1)
    st = workload.build(wl, DEV)
    ne = [wl.n] * wl.B
    res = _run(wl, st, 2048, 512, (1,))
    (o, i, p), r = res
    for b in (0, 63):
        one = ((o[b:b + 1], i[b:b + 1], p[b:b + 1]),
               {l: (x[b:b + 1], y[b:b + 1]) for l, (x, y) in r.items()})
        _check_group_one(wl, st, b, ne[b], 2048, 512, one)


def test_group_1m_sampled():
    """The decoder Full layer at the 1M limit with m = 1 (8 sequences x
    1,048,576 entries): its own top-512 over every visible position and the
    pool of 2,048 blocks of 8 (131,072 block maxima) both take the
    two-stage selection; one Reindex layer on the pool; sequences 0 and 7
    checked."""
    wl = dataclasses.replace(WORKLOADS[4], pool=None, reuse_layers=1)
    st = workload.build(wl, DEV)
    res = _run(wl, st, 2048, 512, (1,))
    (o, i, p), r = res
    for b in (0, wl.B - 1):
        one = ((o[b:b + 1], i[b:b + 1], p[b:b + 1]),
               {l: (x[b:b + 1], y[b:b + 1]) for l, (x, y) in r.items()})
        _check_group_one(wl, st, b, wl.n, 2048, 512, one)


def _check_group_one(wl, st, b, n, n_keep, k, res):
    """The checks of _check_group for one sequence b whose results sit at
    index 0."""
    (out0, ids0, pool), reidx = res
    y = inputs.idx_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
    ic, isc = O.pack_idx(y)
    qi, w = inputs.index_query(wl, b, DEV)
    sc = O.indexer_scores(bf16_bits(qi), w.cpu().numpy(),
                          O.unpack_idx(ic[:n], isc[:n]))
    ok, msg = topk_set_ok(ids0[0], sc, k)
    assert ok, (b, "full", msg)
    _attn_ok(wl, st, b, 0, ids0[0], out0[0])
    bs = O.block_max_scores(sc, n, 8)
    gp = pool[0]
    gv = gp[gp >= 0]
    assert np.all(np.diff(gv) > 0)
    if O.topk_gap(bs, n_keep) >= GAP_TOL:
        assert np.array_equal(gp, O.hier_pool(bs, n, n_keep, 8)), b
    else:
        thr = np.sort(bs)[::-1][n_keep - 1]
        assert np.all(bs[np.unique(gv // 8)] >= thr * (1 - GAP_TOL)), b
    for layer, (out_l, ids_l) in reidx.items():
        qi_l, w_l = inputs.index_query(wl, b, DEV, layer=layer)
        fine = O.indexer_scores(bf16_bits(qi_l), w_l.cpu().numpy(),
                                O.unpack_idx(ic[gv], isc[gv]))
        ok, msg_l = topk_set_ok(ids_l[0], fine, k, ids=gv)
        assert ok, (b, layer, msg_l)
        _attn_ok(wl, st, b, layer, ids_l[0], out_l[0])
    print(b, msg, flush=True)


def test_reindex_crowded_pool_fallback():
    """A pool whose first candidate group holds 200 copies of the row's best
    indexer key (far more than a group keeps): the pool's candidates cannot
    hold the top k, so the exact fallback over the pool decides, with the
    pool's entry ids; the copies tie and the lower ids win.  Pool positions
    are every other entry from 1 (ascending), with a tail of -1 padding."""
    wl = dataclasses.replace(WORKLOADS[2], cid=305, B=2, n=30000)
    st = workload.build(wl, DEV)
    k, n_pool = 512, 12000
    pool = np.full((wl.B, n_pool), -1, np.int32)
    pool[:, :11000] = np.arange(11000, dtype=np.int32) * 2 + 1
    ids_planted = pool[0, 40:240]
    for b in range(wl.B):
        ic = st.idx_codes[b].cpu().numpy()
        isc = st.idx_scales[b].cpu().numpy()
        sc = O.indexer_scores(bf16_bits(st.q_idx[b]), st.w[b].cpu().numpy(),
                              O.unpack_idx(ic[pool[b, :11000]],
                                           isc[pool[b, :11000]]))
        best = int(pool[b, int(np.argmax(sc))])
        rows = torch.from_numpy(ids_planted.astype(np.int64)).to(DEV)
        st.idx_codes[b, rows] = st.idx_codes[b, best].clone()
        st.idx_scales[b, rows] = st.idx_scales[b, best].clone()
    pool_t = torch.from_numpy(pool).to(DEV)
    out, ids = csa2.reindex_decode(st.cache, pool_t, st.q_idx, st.w, st.q[0],
                                   st.swa[0], st.n_swa, k, st.scale)
    torch.cuda.synchronize()
    out, ids = out.float().cpu().numpy(), ids.cpu().numpy()
    for b in range(wl.B):
        gv = pool[b, :11000]
        ic = st.idx_codes[b].cpu().numpy()
        isc = st.idx_scales[b].cpu().numpy()
        fine = O.indexer_scores(bf16_bits(st.q_idx[b]), st.w[b].cpu().numpy(),
                                O.unpack_idx(ic[gv], isc[gv]))
        ok, msg = topk_set_ok(ids[b], fine, k, ids=gv)
        assert ok, (b, msg)
        assert set(ids_planted.tolist()) <= set(ids[b].tolist()), b
        e = _attn_ok(wl, st, b, 0, ids[b], out[b])
        print(b, msg, f"rel-L2 {e:.2e}", flush=True)
