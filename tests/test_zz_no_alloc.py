"""csa2_sparse_attn_decode_noalloc (the decode without a workspace, on the
library's fixed scratch array) against csa2_sparse_attn_decode with a
workspace: bit-equal outputs and top-k ids on two calls in a row, the second
with a smaller input, plus the size limit (rejected before any launch) and
the oracle's top-k rule on one sequence of each call."""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2, workload
from fp4_kv_cache_amd.inputs import WORKLOADS
from _util import bf16_bits, topk_set_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH = 32 << 20


def _both(st):
    """(noalloc out, ids), (workspace out, ids) for the same decode."""
    wl = st.wl
    na = csa2.sparse_attn_decode_noalloc(st.cache, st.q_idx, st.w, st.q[0],
                                         st.swa[0], st.n_swa, wl.k, st.scale)
    ref = csa2.sparse_attn_decode(st.cache, st.q_idx, st.w, st.q[0],
                                  st.swa[0], st.n_swa, wl.k, st.scale)
    torch.cuda.synchronize()
    return na, ref


def _oracle_topk(st, b):
    wl = st.wl
    ic = st.idx_codes[b].cpu().numpy()
    isc = st.idx_scales[b].cpu().numpy()
    sc = O.indexer_scores(bf16_bits(st.q_idx[b]), st.w[b].cpu().numpy(),
                          O.unpack_idx(ic, isc))
    return sc


def test_noalloc_matches_workspace_call_twice():
    big = dataclasses.replace(WORKLOADS[1], cid=301, B=6, n=30000)
    small = dataclasses.replace(WORKLOADS[1], cid=302, B=2, n=7000)
    for wl in (big, small):
        st = workload.build(wl, DEV)
        need = csa2.workspace_size(csa2.OP_DECODE, wl.B, wl.n, wl.k)
        assert need <= SCRATCH
        (o1, i1), (o2, i2) = _both(st)
        assert torch.equal(i1, i2), wl.name
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        ids = i1.cpu().numpy()
        ok, msg = topk_set_ok(ids[0], _oracle_topk(st, 0), wl.k)
        assert ok, msg


def test_noalloc_rejects_calls_beyond_its_scratch():
    wl = dataclasses.replace(WORKLOADS[1], cid=303, B=1, n=1000)
    st = workload.build(wl, DEV)
    L = csa2.load()
    need = csa2.workspace_size(csa2.OP_DECODE, 64, 1 << 20, 512)
    assert need > SCRATCH
    desc = csa2.cache_desc(st.main_codes, st.main_scales, st.idx_codes,
                           st.idx_scales, st.n_entries)
    desc.n_cap = 1 << 20          # never read: rejected before any launch
    out = torch.empty((64, 64, 512), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((64, 512), dtype=torch.int32, device=DEV)
    st_ = L.csa2_sparse_attn_decode_noalloc(
        ctypes.byref(desc), st.q_idx.data_ptr(), st.w.data_ptr(),
        st.q[0].data_ptr(), st.swa[0].data_ptr(), st.n_swa.data_ptr(), 64,
        512, ctypes.c_float(st.scale), None, out.data_ptr(), ids.data_ptr(),
        None)
    assert st_ == 4, st_                     # CSA2_ERR_WORKSPACE
    assert "scratch" in L.csa2_last_error().decode()
