"""The decode path's fused selection against the oracle: each attention
workgroup selects its sequence's top-k from the indexer's per-workgroup
local candidates, falling back to the exact streaming selection over the
whole key row when the candidates cannot be shown to hold the top k.

Cases: sequences whose winners are spread (the candidate path), all-equal
scores (every group ties at its bound: fallback), one group holding far
more winners than it keeps (fallback), rows shorter than k, a 64-row
batch with ragged rows and the fallback over it, the top-k ids
written to topk_out by the same call, and every split count the attention
plans, each sequence of the batch checked, twice in a row on the same
workspace."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2, inputs, workload
from fp4_kv_cache_amd.inputs import WORKLOADS
from _util import (REL_L2_TOL, bf16_bits, planned_splits, rel_l2,
                   split_parts_bytes, topk_set_ok)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(st, b):
    wl = st.wl
    mc = st.main_codes[b].cpu().numpy()
    ms = st.main_scales[b].cpu().numpy()
    ic = st.idx_codes[b].cpu().numpy()
    isc = st.idx_scales[b].cpu().numpy()
    sw = st.swa[0][b].cpu().numpy()
    return mc, ms, ic, isc, sw


def _decode(st, q_idx=None):
    qi = st.q_idx if q_idx is None else q_idx
    out, ids = csa2.sparse_attn_decode(st.cache, qi, st.w, st.q[0],
                                       st.swa[0], st.n_swa, st.wl.k, st.scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), ids.cpu().numpy()


def _check(st, out, ids, b, n, q_idx=None, exact_ids=False):
    mc, ms, ic, isc, sw = _host(st, b)
    qi = bf16_bits((st.q_idx if q_idx is None else q_idx)[b])
    w = st.w[b].cpu().numpy()
    q = bf16_bits(st.q[0][b])
    sel, ref, sc = O.full_layer(mc, ms, ic, isc, n, qi, w, q, sw,
                                st.wl.n_swa, st.wl.k, st.scale)
    if exact_ids:
        assert np.array_equal(ids[b], sel), b
    ok, msg = topk_set_ok(ids[b], sc, st.wl.k)
    assert ok, (b, msg)
    if np.array_equal(ids[b], sel):
        e = rel_l2(out[b], ref)
        assert e <= REL_L2_TOL, (b, e)
    return msg


def test_fused_select_spread_winners():
    """Several groups per row, ragged row lengths (including a row shorter
    than k and an empty one)."""
    wl = dataclasses.replace(WORKLOADS[1], cid=201, B=5, n=12000)
    st = workload.build(wl, DEV)
    ne = [12000, 11111, 4097, 300, 0]
    st.n_entries.copy_(torch.tensor(ne, dtype=torch.int32))
    out, ids = _decode(st)
    for b in range(wl.B):
        if ne[b] == 0:
            assert np.all(ids[b] == -1)
            continue
        print(b, _check(st, out, ids, b, ne[b]))
        assert np.all(ids[b][ids[b] >= 0] < ne[b])


def test_fused_select_all_equal_scores():
    """A zero indexer query scores every entry 0: every group ties at its
    bound, the exact fallback runs, and the lowest k ids win."""
    wl = dataclasses.replace(WORKLOADS[1], cid=202, B=2, n=9000)
    st = workload.build(wl, DEV)
    qz = torch.zeros_like(st.q_idx)
    out, ids = _decode(st, qz)
    for b in range(wl.B):
        assert ids[b].tolist() == list(range(wl.k))
        _check(st, out, ids, b, wl.n, q_idx=qz, exact_ids=True)


def test_fused_select_crowded_group():
    """200 copies of the row's best indexer key inside the first group (far
    more than the group keeps): the candidates cannot hold the top k, so
    the fallback decides; the copies tie and the lower ids win."""
    wl = dataclasses.replace(WORKLOADS[1], cid=203, B=2, n=20000)
    st = workload.build(wl, DEV)
    for b in range(wl.B):
        _, _, ic, isc, _ = _host(st, b)
        sc = O.indexer_scores(bf16_bits(st.q_idx[b]), st.w[b].cpu().numpy(),
                              O.unpack_idx(ic, isc))
        best = int(np.argmax(sc))
        rows = torch.arange(100, 300, device=DEV)
        st.idx_codes[b, rows] = st.idx_codes[b, best].clone()
        st.idx_scales[b, rows] = st.idx_scales[b, best].clone()
    out, ids = _decode(st)
    for b in range(wl.B):
        print(b, _check(st, out, ids, b, wl.n))
        assert set(range(100, 300)) <= set(ids[b].tolist())


def test_fused_select_full_generation_batch():
    """A batch of 64 rows of 16,384 entries (one full generation of scan
    workgroups on 256 CUs), ragged rows, sampled sequences against the
    oracle; then a zero indexer query, where every group ties at its bound
    and the exact fallback reads the key row the scan wrote."""
    n, B = 16384, 64
    wl = dataclasses.replace(WORKLOADS[1], cid=204, B=B, n=n)
    st = workload.build(wl, DEV)
    ne = np.full(B, n, dtype=np.int32)
    ne[1], ne[2], ne[3], ne[B - 2] = n - 1000, 5000, 300, 9173
    st.n_entries.copy_(torch.from_numpy(ne))
    sample = sorted({0, 1, 2, 3, 5, B // 4, B // 2, 3 * B // 4, B - 2, B - 1})
    out, ids = _decode(st)
    for b in sample:
        print(b, _check(st, out, ids, b, int(ne[b])))
        assert np.all(ids[b][ids[b] >= 0] < ne[b])
    qz = torch.zeros_like(st.q_idx)
    out, ids = _decode(st, qz)
    for b in sample[:4] + [B - 1]:
        assert ids[b].tolist() == list(range(min(wl.k, int(ne[b])))) + \
            [-1] * max(0, wl.k - int(ne[b])), b
        _check(st, out, ids, b, int(ne[b]), q_idx=qz, exact_ids=True)


@pytest.mark.parametrize("case", range(10))
def test_fused_decode_random_shapes(case):
    """Seeded random shapes: batch 1-40, 1-6,000 entries, k a multiple of
    16 up to 1,024, window lengths 0-128 per sequence, ragged entry counts
    (including empty rows and rows shorter than k); every sequence against
    the oracle."""
    rng = np.random.default_rng(9000 + case)
    B = int(rng.integers(1, 41))
    n = int(rng.integers(1, 6001))
    k = 16 * int(rng.integers(1, 65))
    wl = dataclasses.replace(WORKLOADS[1], cid=300 + case, B=B, n=n, k=k)
    st = workload.build(wl, DEV)
    ne = rng.integers(0, n + 1, B).astype(np.int32)
    ne[0] = n
    st.n_entries.copy_(torch.from_numpy(ne))
    ns = rng.integers(0, 129, B).astype(np.int32)
    st.n_swa.copy_(torch.from_numpy(ns))
    wl_ns = [int(x) for x in ns]
    out, ids = _decode(st)
    for b in range(B):
        if ne[b] == 0:
            assert np.all(ids[b] == -1), b
        mc, ms, ic, isc, sw = _host(st, b)
        qi = bf16_bits(st.q_idx[b])
        w = st.w[b].cpu().numpy()
        q = bf16_bits(st.q[0][b])
        sel, ref, sc = O.full_layer(mc, ms, ic, isc, int(ne[b]), qi, w, q, sw,
                                    wl_ns[b], k, st.scale)
        ok, msg = topk_set_ok(ids[b], sc, k)
        assert ok, (case, b, msg)
        if ne[b] == 0 and wl_ns[b] == 0:
            continue                      # no key at all: nothing to attend
        if np.array_equal(ids[b], sel):
            e = rel_l2(out[b], ref)
            assert e <= REL_L2_TOL, (case, b, e)
    print(case, B, n, k, "ok", flush=True)


def _split_shape(S):
    best = None
    for B in range(1, 257):
        for k in (64, 96, 128, 160, 192, 224, 256, 288, 384, 512, 768, 1024,
                  1536, 2048):
            if planned_splits(B, k) == S and (best is None or
                                              B * k < best[0] * best[1]):
                best = (B, k)
    return best


@pytest.mark.parametrize("S", [2, 3, 4, 6, 7, 8, 9, 10, 12, 16])
def test_fused_decode_every_split_count(S):
    """The decode call at a batch and k the split planner maps to S splits
    (confirmed through the attention part of the workspace), every sequence
    against the oracle; the call runs twice on one workspace and must give
    the same bits."""
    B, k = _split_shape(S)
    n = max(4 * k, 4096)
    wl = dataclasses.replace(WORKLOADS[1], cid=210 + S, B=B, n=n, k=k)
    st = workload.build(wl, DEV)
    ws_b = csa2.workspace_size(csa2.OP_REUSE, B, n, k)
    assert ws_b == split_parts_bytes(B, S), (B, k, ws_b)
    ws = csa2.workspace(csa2.workspace_size(csa2.OP_DECODE, B, n, k), DEV)
    res = []
    for _ in range(2):
        out, ids = csa2.sparse_attn_decode(st.cache, st.q_idx, st.w, st.q[0],
                                           st.swa[0], st.n_swa, k, st.scale,
                                           ws=ws)
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy(), ids.cpu().numpy()))
    assert np.array_equal(res[0][1], res[1][1])
    assert np.array_equal(res[0][0], res[1][0])
    out, ids = res[1]
    for b in range(B):
        _check(st, out, ids, b, n)
