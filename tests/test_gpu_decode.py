"""End-to-end decode through csa2_sparse_attn_decode (Full layer, and the
hierarchical pool) and the Reuse layers of a decoder group, against the
oracle on the same seeded inputs.

Top-k sets follow the gap rule; attention is compared at rel-L2 <= 5e-3 on
the oracle's own id set (where near-ties let the sets differ, the GPU
attention is re-run on the oracle's ids through the Reuse call)."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_amd import csa2, inputs, workload
from fp4_kv_cache_amd.inputs import WORKLOADS
from _util import REL_L2_TOL, bf16_bits, rel_l2, topk_set_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_caches(wl, b):
    """Oracle-packed caches of sequence b (drawn on the GPU, as the GPU side
    was, and copied to the host)."""
    x = inputs.main_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
    y = inputs.idx_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
    mc, ms = O.pack_main(x)
    ic, isc = O.pack_idx(y)
    return mc, ms, ic, isc


def _oracle_query(wl, b, layer=0):
    qi, w = inputs.index_query(wl, b, DEV)
    q = inputs.attn_query(wl, b, layer, DEV)
    sw = O.pack_swa(inputs.window_latents(wl, b, layer, DEV).cpu().numpy())
    return bf16_bits(qi), w.cpu().numpy(), bf16_bits(q), sw


def _check_seq(st, b, out, ids, layer_outs=()):
    wl = st.wl
    mc, ms, ic, isc = _oracle_caches(wl, b)
    # The GPU pack of this sequence must match the oracle's bytes.
    assert np.array_equal(st.idx_codes[b].cpu().numpy(), ic)
    assert np.array_equal(st.main_scales[b].cpu().numpy(), ms)
    qi, w, q, sw = _oracle_query(wl, b)
    if wl.pool is None:
        sel, ref, sc = O.full_layer(mc, ms, ic, isc, wl.n, qi, w, q, sw,
                                    wl.n_swa, wl.k, st.scale)
        ok, msg = topk_set_ok(ids[b], sc, wl.k)
    else:
        bk = O.block_keys(ic, isc, wl.n, wl.pool[1])
        assert np.array_equal(
            st.block_keys[b].cpu().view(torch.int16).numpy().view(np.uint16)
            [:bk.shape[0]], bk)
        sel, ref, pool, fine = O.hier_layer(
            mc, ms, ic, isc, bk, wl.n, qi, w, q, sw, wl.n_swa, wl.k, st.scale,
            n_keep=wl.pool[0], block=wl.pool[1])
        ok, msg = topk_set_ok(ids[b], fine, wl.k, ids=pool[pool >= 0])
    assert ok, (b, msg)
    got = out[b]
    if not np.array_equal(ids[b], sel):
        # near-tie: rerun the GPU attention on the oracle's ids
        t = torch.from_numpy(np.ascontiguousarray(sel[None]).astype(
            np.int32)).to(DEV)
        got = csa2.reuse_attn(st.main_codes[b:b + 1], st.main_scales[b:b + 1],
                              t, st.q[0][b:b + 1], st.swa[0][b:b + 1],
                              st.n_swa[b:b + 1], st.scale)[0].float().cpu().numpy()
    e = rel_l2(got, ref)
    assert e <= REL_L2_TOL, (b, e)
    errs = [e]
    for layer, lo in enumerate(layer_outs, start=1):
        _, _, ql, swl = _oracle_query(wl, b, layer)
        r = O.reuse_layer(mc, ms, ids[b], ql, swl, wl.n_swa, st.scale)
        el = rel_l2(lo[b], r)
        assert el <= REL_L2_TOL, (b, layer, el)
        errs.append(el)
    return msg, errs


def _run(st):
    out, ids = csa2.sparse_attn_decode(st.cache, st.q_idx, st.w, st.q[0],
                                       st.swa[0], st.n_swa, st.wl.k, st.scale,
                                       pool=st.wl.pool)
    reuse = [csa2.reuse_attn(st.main_codes, st.main_scales, ids, st.q[l],
                             st.swa[l], st.n_swa, st.scale)
             for l in range(1, 1 + st.wl.reuse_layers)]
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), ids.cpu().numpy(),
            [r.float().cpu().numpy() for r in reuse])


def test_tiny_config_all_sequences():
    st = workload.build(WORKLOADS[0], DEV)
    out, ids, _ = _run(st)
    for b in range(st.wl.B):
        msg, errs = _check_seq(st, b, out, ids)
        print(b, msg, errs)


@pytest.mark.parametrize("variant", ["ragged", "pool", "group"])
def test_small_variants(variant):
    if variant == "ragged":
        wl = dataclasses.replace(WORKLOADS[1], cid=101, B=3, n=20000)
    elif variant == "pool":
        wl = dataclasses.replace(WORKLOADS[4], cid=104, B=2, n=8 * 4000 + 5,
                                 pool=(256, 8))
    else:
        wl = dataclasses.replace(WORKLOADS[2], cid=102, B=2, n=9000)
    st = workload.build(wl, DEV)
    out, ids, reuse = _run(st)
    for b in range(wl.B):
        msg, errs = _check_seq(st, b, out, ids, reuse)
        print(variant, b, msg, errs)


def test_ragged_n_entries_in_one_batch():
    wl = dataclasses.replace(WORKLOADS[1], cid=105, B=3, n=6000)
    st = workload.build(wl, DEV)
    ne = [6000, 2500, 300]
    st.n_entries.copy_(torch.tensor(ne, dtype=torch.int32))
    out, ids, _ = _run(st)
    for b in range(3):
        mc, ms, ic, isc = _oracle_caches(wl, b)
        qi, w, q, sw = _oracle_query(wl, b)
        sel, ref, sc = O.full_layer(mc, ms, ic, isc, ne[b], qi, w, q, sw,
                                    wl.n_swa, wl.k, st.scale)
        ok, msg = topk_set_ok(ids[b], sc, wl.k)
        assert ok, (b, msg)
        assert np.all(ids[b][ids[b] >= 0] < ne[b])
        if np.array_equal(ids[b], sel):
            assert rel_l2(out[b], ref) <= REL_L2_TOL


def test_pool_crowded_block_group_fallback():
    """The hierarchical decode with 300 copies of a sequence's best block
    key planted in blocks 200 .. 499 (far more than the block scan's
    candidate group of those rows keeps): the block candidates cannot hold
    the top 2,048 blocks, so the block selection's exact fallback decides.
    The oracle runs the pages' hierarchy on the same (planted) block keys."""
    wl = dataclasses.replace(WORKLOADS[4], cid=106, B=2, n=8 * 16384,
                             pool=(2048, 8))
    st = workload.build(wl, DEV)
    planted = np.arange(200, 500)
    for b in range(wl.B):
        bk = st.block_keys[b].cpu().view(torch.int16).numpy().view(np.uint16)
        qi = bf16_bits(st.q_idx[b])
        bs = O.indexer_scores(qi, st.w[b].cpu().numpy(),
                              F.bf16_bits_to_f64(bk[:16384]))
        best = int(np.argmax(bs))
        rows = torch.from_numpy(planted.astype(np.int64)).to(DEV)
        st.block_keys[b, rows] = st.block_keys[b, best].clone()
    out, ids, _ = _run(st)
    for b in range(wl.B):
        mc, ms, ic, isc = _oracle_caches(wl, b)
        qi, w, q, sw = _oracle_query(wl, b)
        bk = st.block_keys[b].cpu().view(torch.int16).numpy().view(np.uint16)
        bk = bk[:16384]
        sel, ref, pool, fine = O.hier_layer(
            mc, ms, ic, isc, bk, wl.n, qi, w, q, sw, wl.n_swa, wl.k,
            st.scale, n_keep=2048, block=8)
        blocks = set((pool[pool >= 0] // 8).tolist())
        assert set(planted.tolist()) <= blocks, b
        ok, msg = topk_set_ok(ids[b], fine, wl.k, ids=pool[pool >= 0])
        assert ok, (b, msg)
        if np.array_equal(ids[b], sel):
            e = rel_l2(out[b], ref)
            assert e <= REL_L2_TOL, (b, e)
        print(b, msg, flush=True)


@pytest.mark.parametrize("case", range(6))
def test_pool_decode_random_shapes(case):
    """Seeded random hierarchical decodes: batch 1-6, 3,000-40,000 entries
    (ragged last block), pools of 128-2,048 blocks of 8, k a multiple of 16
    below the pool's positions; every sequence against the oracle's
    hierarchy (block keys bit for bit, pool, top-k by the gap rule,
    attention)."""
    rng = np.random.default_rng(9100 + case)
    B = int(rng.integers(1, 7))
    n = int(rng.integers(3000, 40001))
    n_keep = int(rng.choice([128, 512, 1024, 2048]))
    k = 16 * int(rng.integers(1, 33))
    k = min(k, (n_keep * 8) // 2)
    wl = dataclasses.replace(WORKLOADS[4], cid=400 + case, B=B, n=n, k=k,
                             pool=(n_keep, 8))
    st = workload.build(wl, DEV)
    out, ids, _ = _run(st)
    for b in range(B):
        msg, errs = _check_seq(st, b, out, ids)
        print(case, B, n, n_keep, k, b, msg, errs, flush=True)
