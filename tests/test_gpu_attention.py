"""GPU gather-dequant attention (the Reuse-layer call) against the oracle,
fed the same top-k ids: relative L2 <= 5e-3 per sequence."""
import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2
from fp4_kv_cache_amd.workload import attn_scale
from _util import REL_L2_TOL, bf16_bits, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(B, n_cap, k, seed, n_swa):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B * n_cap, 512)).astype(np.float32)
    mc, ms = csa2.pack_kv(csa2.FMT_MAIN, torch.from_numpy(x).to(DEV))
    sw = rng.standard_normal((B * 128, 512)).astype(np.float32)
    swc, _ = csa2.pack_kv(csa2.FMT_SWA, torch.from_numpy(sw).to(DEV))
    q = torch.from_numpy(rng.standard_normal((B, 64, 512)).astype(np.float32))
    q = q.to(torch.bfloat16).to(DEV)
    ids = np.full((B, k), -1, np.int32)
    for b in range(B):
        cnt = min(k, n_cap) - (b % 3) * 5          # some -1 padding
        cnt = max(cnt, 1)
        ids[b, :cnt] = np.sort(rng.choice(n_cap, cnt, replace=False))
    return (mc.view(B, n_cap, 256), ms.view(B, n_cap, 32),
            swc.view(B, 128, 512), q, ids,
            torch.tensor(n_swa, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("B,n_cap,k", [(1, 700, 512), (5, 3000, 512),
                                       (64, 600, 512), (3, 300, 64),
                                       (2, 5000, 2048)])
def test_reuse_attention_vs_oracle(B, n_cap, k):
    n_swa = [128 if b % 4 else (b * 37) % 129 for b in range(B)]
    mc, ms, sw, q, ids, nsw = _setup(B, n_cap, k, B * 1000 + k, n_swa)
    out = csa2.reuse_attn(mc, ms, torch.from_numpy(ids).to(DEV), q, sw, nsw,
                          attn_scale())
    got = out.float().cpu().numpy()
    mcc, msc, swc = mc.cpu().numpy(), ms.cpu().numpy(), sw.cpu().numpy()
    worst = 0.0
    for b in range(B):
        if (ids[b] >= 0).sum() + n_swa[b] == 0:
            continue
        ref = O.reuse_layer(mcc[b], msc[b], ids[b], bf16_bits(q[b]), swc[b],
                            n_swa[b], attn_scale())
        e = rel_l2(got[b], ref)
        worst = max(worst, e)
        assert e <= REL_L2_TOL, (b, e)
    print(f"worst rel-L2 {worst:.2e}")


def test_attention_is_deterministic():
    mc, ms, sw, q, ids, nsw = _setup(8, 2000, 512, 5, [128] * 8)
    t = torch.from_numpy(ids).to(DEV)
    a = csa2.reuse_attn(mc, ms, t, q, sw, nsw, attn_scale())
    b = csa2.reuse_attn(mc, ms, t, q, sw, nsw, attn_scale())
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
