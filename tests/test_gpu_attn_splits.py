"""Every split count of the attention (2 to 16 workgroups per sequence,
each merged by its own instance of the merge kernel) against the oracle:
for each count, a batch size and k that the split planner maps to it, the
count confirmed through the library's workspace size."""
import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2
from fp4_kv_cache_amd.workload import attn_scale
from _util import (REL_L2_TOL, bf16_bits, planned_splits, rel_l2,
                   split_parts_bytes)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shape_for(S):
    best = None
    for B in range(1, 257):
        for k in (16, 32, 48, 64, 96, 128, 160, 192, 224, 256, 288, 320, 352,
                  384, 448, 512, 640, 768, 1024, 1280, 1536, 2048):
            if planned_splits(B, k) == S and (best is None or
                                              B * k < best[0] * best[1]):
                best = (B, k)
    return best


@pytest.mark.parametrize("S", list(range(2, 17)))
def test_attention_every_split_count(S):
    shape = _shape_for(S)
    assert shape is not None, S
    B, k = shape
    n_cap = max(2 * k, 256)
    ws_bytes = csa2.workspace_size(csa2.OP_REUSE, B, n_cap, k)
    assert ws_bytes == split_parts_bytes(B, S), (B, k, ws_bytes)
    rng = np.random.default_rng(7000 + S)
    x = rng.standard_normal((B * n_cap, 512)).astype(np.float32)
    mc, ms = csa2.pack_kv(csa2.FMT_MAIN, torch.from_numpy(x).to(DEV))
    sw = rng.standard_normal((B * 128, 512)).astype(np.float32)
    swc, _ = csa2.pack_kv(csa2.FMT_SWA, torch.from_numpy(sw).to(DEV))
    q = torch.from_numpy(rng.standard_normal((B, 64, 512)).astype(np.float32))
    q = q.to(torch.bfloat16).to(DEV)
    ids = np.stack([np.sort(rng.choice(n_cap, k, replace=False))
                    for _ in range(B)]).astype(np.int32)
    n_swa = [128 - (b * 29) % 97 for b in range(B)]
    mc, ms = mc.view(B, n_cap, 256), ms.view(B, n_cap, 32)
    swc = swc.view(B, 128, 512)
    out = csa2.reuse_attn(mc, ms, torch.from_numpy(ids).to(DEV), q, swc,
                          torch.tensor(n_swa, dtype=torch.int32, device=DEV),
                          attn_scale())
    got = out.float().cpu().numpy()
    mcc, msc, swh = mc.cpu().numpy(), ms.cpu().numpy(), swc.cpu().numpy()
    for b in sorted({0, B - 1}):
        ref = O.reuse_layer(mcc[b], msc[b], ids[b], bf16_bits(q[b]), swh[b],
                            n_swa[b], attn_scale())
        e = rel_l2(got[b], ref)
        assert e <= REL_L2_TOL, (S, B, k, b, e)
