"""GPU gather-dequant attention (the Reuse-layer call) against the oracle,
fed the same top-k ids: relative L2 <= 5e-3 per sequence."""
import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2
from fp4_kv_cache_amd.workload import attn_scale
from _util import REL_L2_TOL, bf16_bits, head_rel_l2_max, rel_l2

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
    worst = head = 0.0
    for b in range(B):
        if (ids[b] >= 0).sum() + n_swa[b] == 0:
            continue
        ref = O.reuse_layer(mcc[b], msc[b], ids[b], bf16_bits(q[b]), swc[b],
                            n_swa[b], attn_scale())
        e = rel_l2(got[b], ref)
        worst = max(worst, e)
        head = max(head, head_rel_l2_max(got[b], ref))
        assert e <= REL_L2_TOL, (b, e)
    print(f"worst rel-L2 {worst:.2e}; worst per-head rel-L2 {head:.2e}")


def test_attention_extreme_ranges():
    """Entries at the FP4 limit (E2M1 6 x E4M3 448 = 2688) and window rows at
    the E4M3 limit (448), with queries spanning bf16's range: heads scaled
    by 3e5 (a one-hot softmax), 1e4, 1e-6 and 1e-30, a head of zeros and
    heads mixing 1e3 and 1e-3 values.  Each head's prescale keeps its fp16
    products exact, so every head stays within the tolerance."""
    rng = np.random.default_rng(4242)
    B, n_cap, k = 2, 2000, 512
    x = rng.standard_normal((B * n_cap, 512)).astype(np.float32)
    g = x.reshape(-1, 32, 16)
    big = rng.choice(B * n_cap, 300, replace=False)
    g[big] = g[big] / np.abs(g[big]).max(axis=2, keepdims=True) * 2688.0
    tiny = rng.choice(B * n_cap, 200, replace=False)
    g[tiny] *= 1e-3
    mc, ms = csa2.pack_kv(csa2.FMT_MAIN, torch.from_numpy(x).to(DEV))
    sw = rng.standard_normal((B * 128, 512)).astype(np.float32)
    sw[::5] = np.clip(sw[::5] * 200.0, -448.0, 448.0)
    swc, _ = csa2.pack_kv(csa2.FMT_SWA, torch.from_numpy(sw).to(DEV))
    qf = rng.standard_normal((B, 64, 512)).astype(np.float32)
    qf[:, 0] *= 3e5
    qf[:, 1] *= 1e4
    qf[:, 2] *= 1e-6
    qf[:, 3] *= 1e-30
    qf[:, 4] = 0.0
    qf[:, 5:9, :256] *= 1e3
    qf[:, 5:9, 256:] *= 1e-3
    q = torch.from_numpy(qf).to(torch.bfloat16).to(DEV)
    ids = np.stack([np.sort(rng.choice(n_cap, k, replace=False))
                    for _ in range(B)]).astype(np.int32)
    # Make sure the limit rows are chosen.
    for b in range(B):
        own = big[(big // n_cap) == b] % n_cap
        ids[b, :len(own[:100])] = np.sort(own[:100])
        ids[b] = np.sort(np.unique(np.concatenate(
            [ids[b], rng.choice(n_cap, k, replace=False)]))[:k])
    n_swa = [128, 77]
    mc3, ms3, sw3 = (mc.view(B, n_cap, 256), ms.view(B, n_cap, 32),
                     swc.view(B, 128, 512))
    out = csa2.reuse_attn(mc3, ms3, torch.from_numpy(ids).to(DEV), q, sw3,
                          torch.tensor(n_swa, dtype=torch.int32, device=DEV),
                          attn_scale())
    got = out.float().cpu().numpy()
    for b in range(B):
        km = O.unpack_main(mc3[b].cpu().numpy(), ms3[b].cpu().numpy())
        assert np.abs(km).max() == 2688.0
        ref = O.reuse_layer(mc3[b].cpu().numpy(), ms3[b].cpu().numpy(),
                            ids[b], bf16_bits(q[b]), sw3[b].cpu().numpy(),
                            n_swa[b], attn_scale())
        assert np.all(np.isfinite(got[b]))
        e = rel_l2(got[b], ref)
        hmax = head_rel_l2_max(got[b], ref)
        print(b, f"rel-L2 {e:.2e}, worst head {hmax:.2e}")
        assert e <= REL_L2_TOL, (b, e)
        assert hmax <= REL_L2_TOL, (b, hmax)


def test_attention_is_deterministic():
    mc, ms, sw, q, ids, nsw = _setup(8, 2000, 512, 5, [128] * 8)
    t = torch.from_numpy(ids).to(DEV)
    a = csa2.reuse_attn(mc, ms, t, q, sw, nsw, attn_scale())
    b = csa2.reuse_attn(mc, ms, t, q, sw, nsw, attn_scale())
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
