"""GPU indexer scores and top-k against the oracle.

Scores: float32 accumulation of exact products, compared with the float64
oracle at a relative tolerance far inside the 1e-5 top-k gap band.
Top-k: both sides select over the SAME float32 score values, so the chosen
ids must be identical (ties included)."""
import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_amd import csa2
from _util import SCORE_RTOL, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _keys(B, n_cap, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B * n_cap, 128)).astype(np.float32)
    c, s = csa2.pack_kv(csa2.FMT_IDX, torch.from_numpy(x).to(DEV))
    return c.view(B, n_cap, 64), s.view(B, n_cap, 4)


def _query(B, seed):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((B, 32, 128)).astype(np.float32))
    w = torch.from_numpy(rng.uniform(0, 1, (B, 32)).astype(np.float32))
    return q.to(torch.bfloat16).to(DEV), w.to(DEV)


def _ref_scores(c, s, qi, w, b, rows):
    keys = O.unpack_idx(c[b, rows], s[b, rows])
    return O.indexer_scores(bf16_bits(qi[b]), w[b].cpu().numpy(), keys)


def test_indexer_scores_ragged():
    B, n_cap = 4, 3000 + 17
    c, s = _keys(B, n_cap, 0)
    qi, w = _query(B, 1)
    n_entries = [n_cap, 1234, 1, 0]
    ne = torch.tensor(n_entries, dtype=torch.int32, device=DEV)
    sc = csa2.indexer_score(csa2.KEYS_MXFP4, c, s, ne, qi, w).cpu().numpy()
    cc, ss = c.cpu().numpy(), s.cpu().numpy()
    for b in range(B):
        n = n_entries[b]
        if n:
            ref = _ref_scores(cc, ss, qi, w, b, np.arange(n))
            np.testing.assert_allclose(sc[b, :n], ref, rtol=SCORE_RTOL,
                                       atol=1e-4)
        assert np.all(np.isneginf(sc[b, n:]))


def test_indexer_candidates_and_bf16_keys():
    B, n_cap = 2, 2048
    c, s = _keys(B, n_cap, 2)
    qi, w = _query(B, 3)
    ne = torch.tensor([n_cap, 1500], dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(4)
    cand = rng.integers(-5, n_cap + 5, (B, 700)).astype(np.int32)
    sc = csa2.indexer_score(csa2.KEYS_MXFP4, c, s, ne, qi, w,
                            cand=torch.from_numpy(cand).to(DEV)).cpu().numpy()
    cc, ss = c.cpu().numpy(), s.cpu().numpy()
    for b, n in enumerate([n_cap, 1500]):
        ok = (cand[b] >= 0) & (cand[b] < n)
        ref = _ref_scores(cc, ss, qi, w, b, cand[b][ok])
        np.testing.assert_allclose(sc[b][ok], ref, rtol=SCORE_RTOL, atol=1e-4)
        assert np.all(np.isneginf(sc[b][~ok]))
    # bf16 block keys
    bk = torch.from_numpy(rng.standard_normal((B, 300, 128)).astype(
        np.float32)).to(torch.bfloat16).to(DEV)
    nb = torch.tensor([300, 77], dtype=torch.int32, device=DEV)
    sb = csa2.indexer_score(csa2.KEYS_BF16, bk, None, nb, qi, w).cpu().numpy()
    for b, n in enumerate([300, 77]):
        ref = O.indexer_scores(bf16_bits(qi[b]), w[b].cpu().numpy(),
                               F.bf16_bits_to_f64(bf16_bits(bk[b, :n])))
        np.testing.assert_allclose(sb[b, :n], ref, rtol=SCORE_RTOL, atol=1e-4)
        assert np.all(np.isneginf(sb[b, n:]))


@pytest.mark.parametrize("ld,k", [(1024, 512), (5000, 1), (40000, 512),
                                  (70000, 2048), (16384, 7)])
def test_topk_exact_vs_oracle(ld, k):
    rng = np.random.default_rng(ld + k)
    B = 3
    sc = rng.standard_normal((B, ld)).astype(np.float32)
    sc[1] = np.round(sc[1] * 4) / 4          # heavy ties
    sc[2, ::7] = -np.inf                     # invalid entries
    sc[2, 3] = np.nan
    nv = [ld, ld - 123, max(1, ld // 3)]
    out = csa2.topk(torch.from_numpy(sc).to(DEV), k,
                    n_valid=torch.tensor(nv, dtype=torch.int32, device=DEV))
    out = out.cpu().numpy()
    for b in range(B):
        s = sc[b, :nv[b]].astype(np.float64)
        ok = np.isfinite(s)
        ref = O.topk(s[ok], k, ids=np.arange(nv[b])[ok])
        assert np.array_equal(out[b], ref), b


def test_topk_pruning_ignores_values_past_n_valid():
    """Stale values past a row's length must not enter the tile maxima: a
    row of 40,000 scores with n_valid = 39,873 (not a multiple of 32), 511
    tiles holding one 1.0 each and 0.0 elsewhere, and 100.0 past n_valid.
    A tile maximum taken over the stale tail would make exactly k tiles
    clear the pruning bound with only 511 valid entries above it; the
    answer is the 511 ones plus the lowest-id zero.  A second row checks
    the same with N(0,1) scores."""
    ld, nvalid, k = 40000, 39873, 512
    rng = np.random.default_rng(77)
    sc = np.zeros((2, ld), np.float32)
    tiles = np.sort(rng.choice(nvalid // 32, 511, replace=False))
    sc[0, tiles * 32 + rng.integers(0, 32, 511)] = 1.0
    sc[1] = rng.standard_normal(ld).astype(np.float32)
    sc[:, nvalid:] = 100.0
    nv = torch.tensor([nvalid, nvalid - 900], dtype=torch.int32, device=DEV)
    out = csa2.topk(torch.from_numpy(sc).to(DEV), k, n_valid=nv).cpu().numpy()
    for b, n in enumerate((nvalid, nvalid - 900)):
        ref = O.topk(sc[b, :n].astype(np.float64), k)
        assert np.array_equal(out[b], ref), b
    assert np.all(out >= 0)


def test_topk_all_equal_and_short_rows():
    sc = np.zeros((2, 3000), np.float32)
    sc[1, :] = 5.0
    nv = torch.tensor([3000, 100], dtype=torch.int32, device=DEV)
    out = csa2.topk(torch.from_numpy(sc).to(DEV), 512, n_valid=nv).cpu().numpy()
    assert out[0].tolist() == list(range(512))
    assert out[1, :100].tolist() == list(range(100))
    assert np.all(out[1, 100:] == -1)


@pytest.mark.parametrize("k", [512, 2048])
def test_topk_pruning_overflows(k):
    """Rows whose tile maxima all tie: every tile is listed, so a row of
    200,000 scores overflows the tile list (6,250 tiles) and one of 100,000
    the candidate store (3,125 tiles, 100,000 candidates); both fall back to
    the streaming select, and the tie rule picks the lowest ids."""
    ld = 200_000
    sc = np.full((3, ld), 1.5, np.float32)
    sc[2, 50_000:] = 2.0                    # the winners sit after the ties
    nv = torch.tensor([ld, 100_000, ld], dtype=torch.int32, device=DEV)
    out = csa2.topk(torch.from_numpy(sc).to(DEV), k, n_valid=nv).cpu().numpy()
    assert out[0].tolist() == list(range(k))
    assert out[1].tolist() == list(range(k))
    assert out[2].tolist() == list(range(50_000, 50_000 + k))


def test_topk_ids_and_block_expansion():
    rng = np.random.default_rng(9)
    B, ld, kb, blk = 2, 20000, 300, 8
    sc = rng.standard_normal((B, ld)).astype(np.float32)
    limit = [ld * blk - 5, 8 * 1000 + 3]
    nv = [ld, 1001]
    out = csa2.topk(torch.from_numpy(sc).to(DEV), kb,
                    n_valid=torch.tensor(nv, dtype=torch.int32, device=DEV),
                    block=blk,
                    limit=torch.tensor(limit, dtype=torch.int32, device=DEV))
    out = out.cpu().numpy()
    for b in range(B):
        blocks = O.topk(sc[b, :nv[b]].astype(np.float64), kb)
        blocks = blocks[blocks >= 0]
        pos = (blocks[:, None] * blk + np.arange(blk)).reshape(-1)
        want = np.where(pos < limit[b], pos, -1)
        assert np.array_equal(out[b, :len(want)], want)
        assert np.all(out[b, len(want):] == -1)
    # explicit ids (ascending with -1 holes), reported instead of positions
    ids = np.sort(rng.choice(10 ** 6, (B, 5000), replace=False), axis=1)
    ids = ids.astype(np.int32)
    ids[:, -40:] = -1
    sc2 = rng.standard_normal((B, 5000)).astype(np.float32)
    out2 = csa2.topk(torch.from_numpy(sc2).to(DEV), 512,
                     ids=torch.from_numpy(ids).to(DEV)).cpu().numpy()
    for b in range(B):
        ok = ids[b] >= 0
        ref = O.topk(sc2[b][ok].astype(np.float64), 512, ids=ids[b][ok])
        assert np.array_equal(out2[b], ref)


def test_indexer_scores_long_scan_sampled():
    """A scan long enough for the 16-tile wavefronts (8 rows of 262,181
    entries: 8,224 wavefronts of 8 tiles, two generations), ragged row
    counts, checked against the oracle on sampled positions (every tile
    position of a wavefront, the row ends) and -inf past each count."""
    B, n_cap = 8, 262144 + 37
    gen = torch.Generator(device=DEV).manual_seed(4242)
    x = torch.randn((B * n_cap, 128), generator=gen, device=DEV)
    c, s = csa2.pack_kv(csa2.FMT_IDX, x)
    del x
    c, s = c.view(B, n_cap, 64), s.view(B, n_cap, 4)
    qi, w = _query(B, 7)
    n_entries = [n_cap, n_cap - 1000, 123457, 1, 0, 262144, 200000, 77]
    ne = torch.tensor(n_entries, dtype=torch.int32, device=DEV)
    sc = csa2.indexer_score(csa2.KEYS_MXFP4, c, s, ne, qi, w).cpu().numpy()
    cc, ss = c.cpu().numpy(), s.cpu().numpy()
    rng = np.random.default_rng(11)
    for b in range(B):
        n = n_entries[b]
        if n:
            rows = np.unique(np.concatenate([
                rng.integers(0, n, 1500),
                np.arange(0, min(n, 512 * 3)),          # whole wavefronts
                np.arange(max(0, n - 300), n)]))        # the row's end
            ref = _ref_scores(cc, ss, qi, w, b, rows)
            np.testing.assert_allclose(sc[b, rows], ref, rtol=SCORE_RTOL,
                                       atol=1e-4)
        assert np.all(np.isneginf(sc[b, n:])), b


def test_topk_two_stage_crowded_chunk_ties_and_ids():
    """Rows long enough for the two-stage selection (chunks of 4,096 keep
    their top few pairs; the row's top k comes from their union when the
    chunks' bounds prove it).  Row 0 crowds 1,500 of its top 2,048 into one
    chunk, far more than a chunk keeps, so the union proves nothing and the
    row streams through the exact selection; row 1's scores tie in steps
    of 0.5 across every chunk boundary; row 2 is ragged (n_valid).  Then
    explicit ids with -1 holes over 12,000 scores."""
    ld, k = 60000, 2048
    rng = np.random.default_rng(31)
    sc = rng.standard_normal((3, ld)).astype(np.float32)
    sc[0, 8192:8192 + 1500] = 10.0 + rng.random(1500).astype(np.float32)
    sc[1] = np.round(sc[1] * 2) / 2
    nv = [ld, ld, 33333]
    out = csa2.topk(torch.from_numpy(sc).to(DEV), k,
                    n_valid=torch.tensor(nv, dtype=torch.int32, device=DEV))
    out = out.cpu().numpy()
    for b in range(3):
        ref = O.topk(sc[b, :nv[b]].astype(np.float64), k)
        assert np.array_equal(out[b], ref), b
    ids = np.sort(rng.choice(10 ** 7, (2, 12000), replace=False), axis=1)
    ids = ids.astype(np.int32)
    ids[:, ::97] = -1
    sc2 = rng.standard_normal((2, 12000)).astype(np.float32)
    out2 = csa2.topk(torch.from_numpy(sc2).to(DEV), 512,
                     ids=torch.from_numpy(ids).to(DEV)).cpu().numpy()
    for b in range(2):
        ok = ids[b] >= 0
        ref = O.topk(sc2[b][ok].astype(np.float64), 512, ids=ids[b][ok])
        assert np.array_equal(out2[b], ref), b
