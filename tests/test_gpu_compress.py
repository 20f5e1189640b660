"""The decode-time write path on the GPU against the oracle: projections C
and Z, the per-channel softmax pooling over the block's m tokens, the
indexer-key projection, and the append into the caches.

C, C_bar and K^I are float32 sums of exact bf16 products and are compared
with the float64 oracle within the float32 accumulation error; the packed
entry and window rows, whose integer codes float32 decides, must equal the
oracle's packing of the GPU's own float32 values bit for bit; rows and slots
the call does not own stay untouched."""
import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_amd import csa2, inputs
from _util import bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


# (2, 3, 9216): nine reduction slices (the epilogue's 16-slice instance);
# (2, 6, 2048): more tokens than the unrolled epilogue instances take.
@pytest.mark.parametrize("B,m,d", [(3, 2, 512), (5, 1, 1040), (2, 4, 7168),
                                   (32, 2, 7168), (2, 3, 9216), (2, 6, 2048)])
def test_compress_append(B, m, d):
    cid = 500 + m
    h = inputs.hidden_states(cid, B, m, d, DEV)
    wkv, wz, wik = inputs.compressor_weights(cid, d, DEV)
    n_cap = 40
    rng = np.random.default_rng(B * 100 + m)
    rows = rng.integers(0, n_cap, B).astype(np.int32)
    rows[0] = n_cap - 1
    if B > 2:
        rows[2] = -1                      # not written
    slots = rng.integers(0, 128, B).astype(np.int32)
    slots[-1] = 126                       # wraps for m > 2
    fill = lambda *shape: torch.full(shape, 0x5A, dtype=torch.uint8, device=DEV)
    mc, ms = fill(B, n_cap, 256), fill(B, n_cap, 32)
    ic, isc = fill(B, n_cap, 64), fill(B, n_cap, 4)
    sw = fill(B, 128, 512)
    cbar, ki, c = csa2.compress_append(
        h, wkv, wz, wik, torch.from_numpy(rows).to(DEV), mc, ms, ic, isc,
        swa=sw, swa_slot=torch.from_numpy(slots).to(DEV), debug=True)
    cbar, ki, c = (t.cpu().numpy() for t in (cbar, ki, c))
    mc, ms, ic, isc, sw = (t.cpu().numpy() for t in (mc, ms, ic, isc, sw))
    hb = bf16_bits(h)
    wb = [bf16_bits(t) for t in (wkv, wz, wik)]
    for b in range(B):
        rc, rcbar, rki = O.compress_block(hb[b], *wb)
        for got, ref in ((c[b], rc), (cbar[b], rcbar), (ki[b], rki)):
            err = np.abs(got.astype(np.float64) - ref).max()
            assert err <= 1e-4 + 1e-5 * np.abs(ref).max(), (b, err)
        if rows[b] >= 0:
            pc, ps = O.pack_main(cbar[b][None])
            assert np.array_equal(mc[b, rows[b]], pc[0])
            assert np.array_equal(ms[b, rows[b]], ps[0])
            qc, qs = O.pack_idx(ki[b][None])
            assert np.array_equal(ic[b, rows[b]], qc[0])
            assert np.array_equal(isc[b, rows[b]], qs[0])
        for i in range(m):
            slot = (slots[b] + i) % 128
            assert np.array_equal(sw[b, slot], O.pack_swa(c[b, i][None])[0])
        others = [r for r in range(n_cap) if r != rows[b]]
        assert np.all(mc[b, others] == 0x5A) and np.all(ic[b, others] == 0x5A)
        used = {(slots[b] + i) % 128 for i in range(m)}
        free = [s for s in range(128) if s not in used]
        assert np.all(sw[b, free] == 0x5A)
    print(B, m, d, "ok", flush=True)


@pytest.mark.parametrize("case", range(6))
def test_compress_append_random_shapes(case):
    """Seeded random write-path shapes: batch 1-8, m 1-16 tokens per
    block, d a multiple of 16 up to 4,096 (ragged last reduction slice),
    random target rows (some out of range, not written) and window slots."""
    rng = np.random.default_rng(9200 + case)
    B = int(rng.integers(1, 9))
    m = int(rng.integers(1, 17))
    d = 16 * int(rng.integers(1, 257))
    cid = 600 + case
    h = inputs.hidden_states(cid, B, m, d, DEV)
    wkv, wz, wik = inputs.compressor_weights(cid, d, DEV)
    n_cap = 24
    rows = rng.integers(-2, n_cap + 2, B).astype(np.int32)
    slots = rng.integers(0, 128, B).astype(np.int32)
    fill = lambda *shape: torch.full(shape, 0x5A, dtype=torch.uint8, device=DEV)
    mc, ms = fill(B, n_cap, 256), fill(B, n_cap, 32)
    ic, isc = fill(B, n_cap, 64), fill(B, n_cap, 4)
    sw = fill(B, 128, 512)
    cbar, ki, c = csa2.compress_append(
        h, wkv, wz, wik, torch.from_numpy(rows).to(DEV), mc, ms, ic, isc,
        swa=sw, swa_slot=torch.from_numpy(slots).to(DEV), debug=True)
    cbar, ki, c = (t.cpu().numpy() for t in (cbar, ki, c))
    mc, ms, ic, isc, sw = (t.cpu().numpy() for t in (mc, ms, ic, isc, sw))
    hb = bf16_bits(h)
    wb = [bf16_bits(t) for t in (wkv, wz, wik)]
    for b in range(B):
        rc, rcbar, rki = O.compress_block(hb[b], *wb)
        for got, ref in ((c[b], rc), (cbar[b], rcbar), (ki[b], rki)):
            err = np.abs(got.astype(np.float64) - ref).max()
            assert err <= 1e-4 + 1e-5 * np.abs(ref).max(), (case, b, err)
        r = int(rows[b])
        if 0 <= r < n_cap:
            pc, ps = O.pack_main(cbar[b][None])
            assert np.array_equal(mc[b, r], pc[0])
            assert np.array_equal(ms[b, r], ps[0])
            qc, qs = O.pack_idx(ki[b][None])
            assert np.array_equal(ic[b, r], qc[0])
            assert np.array_equal(isc[b, r], qs[0])
        others = [x for x in range(n_cap) if x != r]
        assert np.all(mc[b, others] == 0x5A) and np.all(ic[b, others] == 0x5A)
        used = {(int(slots[b]) + i) % 128 for i in range(m)}
        for i in range(m):
            slot = (int(slots[b]) + i) % 128
            assert np.array_equal(sw[b, slot], O.pack_swa(c[b, i][None])[0])
        free = [x for x in range(128) if x not in used]
        assert np.all(sw[b, free] == 0x5A)
    print(case, B, m, d, "ok", flush=True)
