"""The indexer with an MXFP4 query (V4's FP4 indexer query and key) against
the oracle: the GPU packs the bf16 query heads exactly as the oracle does,
scores match the float64 FP4-query oracle within the float32 accumulation
tolerance (MXFP4 keys through the scaled FP4 matrix op, bf16 block keys
through the dequantised query), and whole decodes follow the top-k gap rule
with attention at rel-L2 <= 5e-3 on the GPU's own id set."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_amd import csa2, inputs, workload
from fp4_kv_cache_amd.inputs import WORKLOADS
from _util import (GAP_TOL, REL_L2_TOL, SCORE_RTOL, bf16_bits, rel_l2,
                   topk_set_ok)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _keys(B, n_cap, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B * n_cap, 128)).astype(np.float32)
    c, s = csa2.pack_kv(csa2.FMT_IDX, torch.from_numpy(x).to(DEV))
    return c.view(B, n_cap, 64), s.view(B, n_cap, 4)


def _query(B, seed):
    """bf16 query heads (some sequences scaled far from 1, to move the MX
    exponents), their GPU MXFP4 planes, and the weights."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, 32, 128)).astype(np.float32)
    q *= np.exp2(rng.integers(-8, 9, (B, 1, 1))).astype(np.float32)
    qi = torch.from_numpy(q).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy(rng.uniform(0, 1, (B, 32)).astype(np.float32)).to(DEV)
    qc, qs = csa2.pack_query_fp4(qi)
    return qi, qc, qs, w


def _oracle_query(qi, b):
    return O.pack_idx(F.bf16_bits_to_f64(bf16_bits(qi[b])))


def test_query_pack_matches_oracle():
    qi, qc, qs, _ = _query(5, 1)
    for b in range(5):
        c, s = _oracle_query(qi, b)
        assert np.array_equal(qc[b].cpu().numpy(), c)
        assert np.array_equal(qs[b].cpu().numpy(), s)


def test_fp4q_scores_ragged():
    B, n_cap = 4, 3000 + 17
    c, s = _keys(B, n_cap, 2)
    qi, qc, qs, w = _query(B, 3)
    n_entries = [n_cap, 1234, 1, 0]
    ne = torch.tensor(n_entries, dtype=torch.int32, device=DEV)
    sc = csa2.indexer_score_fp4q(csa2.KEYS_MXFP4, c, s, ne, qc, qs,
                                 w).cpu().numpy()
    cc, ss = c.cpu().numpy(), s.cpu().numpy()
    for b in range(B):
        n = n_entries[b]
        if n:
            oc, os_ = _oracle_query(qi, b)
            ref = O.indexer_scores_fp4q(oc, os_, w[b].cpu().numpy(),
                                        O.unpack_idx(cc[b, :n], ss[b, :n]))
            np.testing.assert_allclose(sc[b, :n], ref, rtol=SCORE_RTOL,
                                       atol=1e-30 + 1e-6 * float(np.abs(ref).max()))
        assert np.all(np.isneginf(sc[b, n:]))


def test_fp4q_candidates_and_bf16_keys():
    B, n_cap = 2, 2048
    c, s = _keys(B, n_cap, 4)
    qi, qc, qs, w = _query(B, 5)
    ne = torch.tensor([n_cap, 1500], dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(6)
    cand = rng.integers(-5, n_cap + 5, (B, 700)).astype(np.int32)
    sc = csa2.indexer_score_fp4q(csa2.KEYS_MXFP4, c, s, ne, qc, qs, w,
                                 cand=torch.from_numpy(cand).to(DEV))
    sc = sc.cpu().numpy()
    cc, ss = c.cpu().numpy(), s.cpu().numpy()
    for b, n in enumerate([n_cap, 1500]):
        ok = (cand[b] >= 0) & (cand[b] < n)
        oc, os_ = _oracle_query(qi, b)
        ref = O.indexer_scores_fp4q(oc, os_, w[b].cpu().numpy(),
                                    O.unpack_idx(cc[b, cand[b][ok]],
                                                 ss[b, cand[b][ok]]))
        np.testing.assert_allclose(sc[b][ok], ref, rtol=SCORE_RTOL,
                                   atol=1e-6 * float(np.abs(ref).max()))
        assert np.all(np.isneginf(sc[b][~ok]))
    bk = torch.from_numpy(rng.standard_normal((B, 300, 128)).astype(
        np.float32)).to(torch.bfloat16).to(DEV)
    nb = torch.tensor([300, 77], dtype=torch.int32, device=DEV)
    sb = csa2.indexer_score_fp4q(csa2.KEYS_BF16, bk, None, nb, qc, qs,
                                 w).cpu().numpy()
    for b, n in enumerate([300, 77]):
        oc, os_ = _oracle_query(qi, b)
        ref = O.indexer_scores_fp4q(oc, os_, w[b].cpu().numpy(),
                                    F.bf16_bits_to_f64(bf16_bits(bk[b, :n])))
        np.testing.assert_allclose(sb[b, :n], ref, rtol=SCORE_RTOL,
                                   atol=1e-6 * float(np.abs(ref).max()))
        assert np.all(np.isneginf(sb[b, n:]))


def _check_decode(st, qc, qs, b, out, ids):
    """Top-k by the gap rule on the oracle's FP4-query scores (flat, or the
    pool of the block scores), then attention on the GPU's ids."""
    wl = st.wl
    n, k = int(st.n_entries[b]), wl.k
    y = inputs.idx_latents(wl, b, 0, wl.n, DEV).cpu().numpy()
    ic, isc = O.pack_idx(y)
    oc, os_ = O.pack_idx(F.bf16_bits_to_f64(bf16_bits(st.q_idx[b])))
    assert np.array_equal(qc[b].cpu().numpy(), oc)
    assert np.array_equal(qs[b].cpu().numpy(), os_)
    w = st.w[b].cpu().numpy()
    g = ids[b]
    gv = g[g >= 0]
    assert len(gv) == min(k, n) and np.all(np.diff(gv) > 0)
    if wl.pool is None:
        sc = O.indexer_scores_fp4q(oc, os_, w, O.unpack_idx(ic[:n], isc[:n]))
        ok, msg = topk_set_ok(g, sc, k)
    else:
        n_keep, block = wl.pool
        bk = O.block_keys(ic, isc, n, block)
        bs = O.indexer_scores_fp4q(oc, os_, w, F.bf16_bits_to_f64(bk))
        kb = min(n_keep, len(bs))
        if O.topk_gap(bs, kb) >= GAP_TOL:
            pool = O.hier_pool(bs, n, n_keep, block)
            valid = pool[pool >= 0]
            fine = O.indexer_scores_fp4q(oc, os_, w,
                                         O.unpack_idx(ic[valid], isc[valid]))
            ok, msg = topk_set_ok(g, fine, k, ids=valid)
        else:
            thr = np.sort(bs)[::-1][kb - 1]
            ok = bool(np.all(bs[np.unique(gv // block)] >= thr * (1 - GAP_TOL)))
            msg = "block near-tie; pool membership checked"
    assert ok, (b, msg)
    sel = torch.from_numpy(gv.astype(np.int64)).to(DEV)
    x = inputs.main_latents(wl, b, 0, wl.n, DEV)[sel].cpu().numpy()
    mc, ms = O.pack_main(x)
    sw = O.pack_swa(inputs.window_latents(wl, b, 0, DEV).cpu().numpy())
    keys = np.concatenate([O.unpack_main(mc, ms),
                           O.unpack_swa(sw[:wl.n_swa])], axis=0)
    ref = O.mqa_decode(bf16_bits(st.q[0][b]), keys, st.scale)
    e = rel_l2(out[b], ref)
    assert e <= REL_L2_TOL, (b, e)
    return msg, e


def _decode(st, ws=None):
    qc, qs = csa2.pack_query_fp4(st.q_idx)
    out, ids = csa2.sparse_attn_decode_fp4q(st.cache, qc, qs, st.w, st.q[0],
                                            st.swa[0], st.n_swa, st.wl.k,
                                            st.scale, pool=st.wl.pool, ws=ws)
    torch.cuda.synchronize()
    return qc, qs, out.float().cpu().numpy(), ids.cpu().numpy()


@pytest.mark.parametrize("variant", ["ragged", "pool"])
def test_fp4q_decode_small(variant):
    if variant == "ragged":
        wl = dataclasses.replace(WORKLOADS[1], cid=201, B=3, n=20000)
    else:
        wl = dataclasses.replace(WORKLOADS[4], cid=204, B=2, n=8 * 4000 + 5,
                                 pool=(256, 8))
    st = workload.build(wl, DEV)
    if variant == "ragged":
        st.n_entries.copy_(torch.tensor([20000, 11111, 700], dtype=torch.int32))
    qc, qs, out, ids = _decode(st)
    for b in range(wl.B):
        msg, e = _check_decode(st, qc, qs, b, out, ids)
        print(variant, b, msg, f"rel-L2 {e:.2e}", flush=True)


def test_fp4q_decode_full_size_sampled():
    """The 64K-context workload at full size (32 sequences x 32,768
    entries), in the benchmark's launch configuration; sequences 0 and 31
    are checked against the oracle."""
    wl = WORKLOADS[1]
    st = workload.build(wl, DEV)
    ws = csa2.workspace(csa2.workspace_size(csa2.OP_DECODE, wl.B, wl.n, wl.k,
                                            wl.pool), DEV)
    qc, qs, out, ids = _decode(st, ws)
    for b in (0, 31):
        msg, e = _check_decode(st, qc, qs, b, out, ids)
        print("full", b, msg, f"rel-L2 {e:.2e}", flush=True)
