"""Parity at the full workload sizes, in the launch configuration the
benchmark times: one csa2_sparse_attn_decode over the whole batch (plus the
three Reuse layers of the decoder group), then sampled sequences checked
one by one against the oracle on the same drawn inputs.

For a sampled sequence b the oracle packs b's indexer keys from the drawn
latents (and must reproduce the GPU's bytes), scores every visible entry in
float64 (or, hierarchically, the block keys and then the pool) and checks the
GPU's top-k set by the gap rule.  The attention output is compared, at
rel-L2 <= 5e-3, with the oracle's attention over the GPU's own id set; only
those main rows are packed on the host, again bit-compared with the GPU's."""
import gc

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_amd import csa2, inputs, workload
from fp4_kv_cache_amd.inputs import WORKLOADS
from _util import (GAP_TOL, REL_L2_TOL, bf16_bits, head_rel_l2_max, rel_l2,
                   topk_set_ok)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SAMPLES = {1: (0, 31), 2: (0, 63), 3: (0, 1, 2, 3), 4: (0, 5)}


def _query(wl, b, layer=0):
    qi, w = inputs.index_query(wl, b, DEV)
    q = inputs.attn_query(wl, b, layer, DEV)
    sw = O.pack_swa(inputs.window_latents(wl, b, layer, DEV).cpu().numpy())
    return bf16_bits(qi), w.cpu().numpy(), bf16_bits(q), sw


def _check_pool_ids(g, bs, n, n_keep, block):
    """Top-k checked inside the pool.  When the block scores leave no near-tie
    at the n_keep boundary the pools must agree and the fine top-k follows
    the gap rule; otherwise every chosen position must lie in a block whose
    score is within the tolerance of the boundary or above it."""
    kb = min(n_keep, len(bs))
    thr = np.sort(bs)[::-1][kb - 1]
    blocks = np.unique(g // block)
    return bool(np.all(bs[blocks] >= thr * (1 - GAP_TOL))), O.topk_gap(bs, kb)


def _check_sequence(st, b, out, ids, reuse):
    wl = st.wl
    n, k = wl.n, wl.k
    y = inputs.idx_latents(wl, b, 0, n, DEV).cpu().numpy()
    ic, isc = O.pack_idx(y)
    del y
    assert np.array_equal(st.idx_codes[b].cpu().numpy(), ic), b
    assert np.array_equal(st.idx_scales[b].cpu().numpy(), isc), b
    qi, w, q, sw = _query(wl, b)
    g = ids[b]
    gv = g[g >= 0]
    assert len(gv) == k and np.all(np.diff(gv) > 0), "ids ascending, full"
    if wl.pool is None:
        sc = O.indexer_scores(qi, w, O.unpack_idx(ic, isc))
        ok, msg = topk_set_ok(g, sc, k)
    else:
        n_keep, block = wl.pool
        bk = O.block_keys(ic, isc, n, block)
        gpu_bk = st.block_keys[b].cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(gpu_bk[:bk.shape[0]], bk), b
        bs = O.indexer_scores(qi, w, F.bf16_bits_to_f64(bk))
        in_pool, bgap = _check_pool_ids(gv, bs, n, n_keep, block)
        assert in_pool, (b, "a chosen position outside every eligible block")
        if bgap >= GAP_TOL:
            pool = O.hier_pool(bs, n, n_keep, block)
            valid = pool[pool >= 0]
            fine = O.indexer_scores(qi, w, O.unpack_idx(ic[valid], isc[valid]))
            ok, msg = topk_set_ok(g, fine, k, ids=valid)
        else:
            ok, msg = True, f"block near-tie (gap {bgap:.3g}); pool membership checked"
    del ic, isc
    assert ok, (b, msg)
    # The GPU's chosen main rows, packed on the host from the same latents.
    sel = torch.from_numpy(gv.astype(np.int64)).to(DEV)
    x = inputs.main_latents(wl, b, 0, n, DEV)[sel].cpu().numpy()
    mc, ms = O.pack_main(x)
    assert np.array_equal(st.main_codes[b][sel].cpu().numpy(), mc), b
    assert np.array_equal(st.main_scales[b][sel].cpu().numpy(), ms), b
    km = O.unpack_main(mc, ms)
    errs = []
    for layer in range(1 + wl.reuse_layers):
        if layer:
            _, _, q, sw = _query(wl, b, layer)
        keys = np.concatenate([km, O.unpack_swa(sw[:wl.n_swa])], axis=0)
        ref = O.mqa_decode(q, keys, st.scale)
        got = out[b] if layer == 0 else reuse[layer - 1][b]
        e = rel_l2(got, ref)
        assert e <= REL_L2_TOL, (b, layer, e)
        errs.append(e)
        errs.append(head_rel_l2_max(got, ref))
    return msg, errs


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_full_size_decode_sampled(cid):
    wl = WORKLOADS[cid]
    print(f"config {cid} {wl.name}: B={wl.B} n={wl.n}", flush=True)
    st = workload.build(wl, DEV)
    ws = csa2.workspace(csa2.workspace_size(csa2.OP_DECODE, wl.B, wl.n, wl.k,
                                            wl.pool), DEV)
    out, ids = csa2.sparse_attn_decode(st.cache, st.q_idx, st.w, st.q[0],
                                       st.swa[0], st.n_swa, wl.k, st.scale,
                                       pool=wl.pool, ws=ws)
    reuse = [csa2.reuse_attn(st.main_codes, st.main_scales, ids, st.q[l],
                             st.swa[l], st.n_swa, st.scale)
             for l in range(1, 1 + wl.reuse_layers)]
    torch.cuda.synchronize()
    out_h = out.float().cpu().numpy()
    ids_h = ids.cpu().numpy()
    reuse_h = [r.float().cpu().numpy() for r in reuse]
    for b in SAMPLES[cid]:
        msg, errs = _check_sequence(st, b, out_h, ids_h, reuse_h)
        print(f"  seq {b}: top-k {msg}; rel-L2, worst head per layer: "
              f"{', '.join(f'{e:.2e}' for e in errs)}", flush=True)
    del st, ws, out, ids, reuse
    gc.collect()
    torch.cuda.empty_cache()
