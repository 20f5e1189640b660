"""GPU packing / dequant / block keys: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_amd import csa2

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _adversarial_main(seed):
    """Groups built so that amax/6 sits exactly on E4M3 values and rounding
    midpoints, and elements sit on every E2M1 threshold (and one ulp off)."""
    rng = np.random.default_rng(seed)
    rows = []
    codes = np.arange(1, 0x7E)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for _ in range(64):
        row = np.zeros(512, np.float32)
        for g in range(32):
            s = F.e4m3_decode(rng.choice(codes))
            grp = np.float32(s) * rng.choice(mids, 16).astype(np.float32)
            kind = rng.integers(4)
            if kind == 1:
                grp = np.nextafter(grp, np.float32(np.inf))
            elif kind == 2:
                grp = np.nextafter(grp, np.float32(0))
            grp[0] = np.float32(6 * s)               # amax/6 == s exactly
            if rng.integers(3) == 0:                 # amax/6 on a midpoint
                nxt = F.e4m3_decode(F.e4m3_encode(s) + 1)
                grp[0] = np.float32(3 * (s + nxt))
            grp *= rng.choice([-1, 1], 16).astype(np.float32)
            row[16 * g:16 * g + 16] = grp
        rows.append(row)
    x = np.stack(rows)
    # plus plain N(0,1), tiny, huge, zeros and negative zeros
    x = np.concatenate([x, rng.standard_normal((200, 512)).astype(np.float32),
                        (rng.standard_normal((8, 512)) * 1e-6).astype(np.float32),
                        (rng.standard_normal((8, 512)) * 5e3).astype(np.float32),
                        np.zeros((2, 512), np.float32),
                        -np.zeros((2, 512), np.float32)])
    return x


def test_pack_main_bit_exact():
    x = _adversarial_main(0)
    c, s = csa2.pack_kv(csa2.FMT_MAIN, torch.from_numpy(x).to(DEV))
    rc, rs = O.pack_main(x)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(c.cpu().numpy(), rc)
    deq = csa2.unpack_kv(csa2.FMT_MAIN, c, s).cpu().numpy()
    ref = O.unpack_main(rc, rs)
    assert np.array_equal(deq.astype(np.float64), ref)
    assert np.array_equal(np.signbit(deq), np.signbit(ref))


def test_pack_idx_bit_exact():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((3000, 128)) *
         np.exp2(rng.integers(-30, 30, (3000, 1)))).astype(np.float32)
    x[5] = 0.0
    x[6] = -0.0
    x[7, :32] = 0.0
    # elements on E2M1 thresholds relative to the block exponent
    x[8, :] = np.float32(2.0 ** -3) * np.tile(
        np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32), 16)
    c, s = csa2.pack_kv(csa2.FMT_IDX, torch.from_numpy(x).to(DEV))
    rc, rs = O.pack_idx(x)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(c.cpu().numpy(), rc)
    deq = csa2.unpack_kv(csa2.FMT_IDX, c, s).cpu().numpy()
    assert np.array_equal(deq.astype(np.float64), O.unpack_idx(rc, rs))


def test_pack_swa_bit_exact():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 512)).astype(np.float32)
    x[0] = np.linspace(-600, 600, 512).astype(np.float32)     # saturation
    vals = np.unique(np.abs(F.e4m3_decode(np.arange(0x7F))))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert len(mids) < 512
    x[1, :len(mids)] = mids
    x[2, :len(mids)] = -mids
    c, _ = csa2.pack_kv(csa2.FMT_SWA, torch.from_numpy(x).to(DEV))
    assert np.array_equal(c.cpu().numpy(), O.pack_swa(x))
    deq = csa2.unpack_kv(csa2.FMT_SWA, c).cpu().numpy()
    assert np.array_equal(deq.astype(np.float64), O.unpack_swa(O.pack_swa(x)))


def test_empty_pack_is_noop():
    x = torch.empty((0, 512), dtype=torch.float32, device=DEV)
    c, s = csa2.pack_kv(csa2.FMT_MAIN, x)
    assert c.shape == (0, 256) and s.shape == (0, 32)


def test_block_keys_bit_exact_ragged():
    rng = np.random.default_rng(3)
    B, n_cap = 3, 8 * 50 + 5
    x = rng.standard_normal((B, n_cap, 128)).astype(np.float32)
    c, s = csa2.pack_kv(csa2.FMT_IDX, torch.from_numpy(x.reshape(-1, 128)).to(DEV))
    c = c.view(B, n_cap, 64)
    s = s.view(B, n_cap, 4)
    n_entries = [n_cap, 8 * 20 + 3, 1]
    ne = torch.tensor(n_entries, dtype=torch.int32, device=DEV)
    bk = csa2.build_block_keys(c, s, ne, 8)
    got = bk.cpu().view(torch.int16).numpy().view(np.uint16)
    cc, ss = c.cpu().numpy(), s.cpu().numpy()
    for b in range(B):
        ref = O.block_keys(cc[b], ss[b], n_entries[b])
        nb = ref.shape[0]
        assert np.array_equal(got[b, :nb], ref)
        assert np.all(got[b, nb:] == 0)
