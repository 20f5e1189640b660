"""Pins of the oracle's decode path: brute force with Python loops on tiny
inputs, hand-computable cases, PyTorch's own float64 attention routine, and
the identities the pages state (sparse = dense when top-k covers every
entry; the hierarchical path = the flat path when the pool covers every
block; a Reuse layer fed a Full layer's top-k reproduces its attention)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import formats as F

SCALE = float(np.float32(1.0 / math.sqrt(512)))


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(
        torch.bfloat16).view(torch.uint16).numpy()


def _case(n, seed, n_swa=128):
    rng = np.random.default_rng(seed)
    main = rng.standard_normal((n, 512)).astype(np.float32)
    idx = rng.standard_normal((n, 128)).astype(np.float32)
    swa = rng.standard_normal((128, 512)).astype(np.float32)
    mc, ms = O.pack_main(main)
    ic, is_ = O.pack_idx(idx)
    return dict(mc=mc, ms=ms, ic=ic, is_=is_, sw=O.pack_swa(swa),
                qi=_bf16(rng.standard_normal((32, 128))),
                w=rng.uniform(0, 1, 32).astype(np.float32),
                q=_bf16(rng.standard_normal((64, 512))), n=n, n_swa=n_swa)


# ------------------------------------------------------------- indexer ----
def test_scores_bruteforce_loops():
    c = _case(6, 0)
    keys = O.unpack_idx(c["ic"], c["is_"])
    q = F.bf16_bits_to_f64(c["qi"])
    got = O.indexer_scores(c["qi"], c["w"], keys)
    for j in range(6):
        tot = 0.0
        for h in range(32):
            dot = math.fsum(float(q[h, d]) * float(keys[j, d])
                            for d in range(128))
            tot += float(c["w"][h]) * max(dot, 0.0)
        assert got[j] == pytest.approx(tot, rel=1e-13, abs=1e-13)


def test_scores_hand_cases():
    keys = np.zeros((3, 128))
    keys[0, 5] = 2.0          # one-hot key
    keys[1, 5] = -2.0         # negative dot for every head -> ReLU 0
    keys[2, 7] = 1.0
    qi = np.zeros((32, 128), np.float32)
    qi[:, 5] = 1.5
    qi[3, 7] = -1.0
    w = np.linspace(0.1, 1.0, 32).astype(np.float32)
    s = O.indexer_scores(_bf16(qi), w, keys)
    assert s[0] == pytest.approx(3.0 * float(np.sum(w.astype(np.float64))))
    assert s[1] == 0.0
    assert s[2] == 0.0        # only head 3 touches dim 7, with a negative dot


def test_scores_permutation_equivariant():
    c = _case(50, 1)
    keys = O.unpack_idx(c["ic"], c["is_"])
    perm = np.random.default_rng(2).permutation(50)
    a = O.indexer_scores(c["qi"], c["w"], keys)
    b = O.indexer_scores(c["qi"], c["w"], keys[perm])
    assert np.array_equal(a[perm], b)


def _e2m1_table():
    """E2M1 magnitudes of codes 0..7 from the cited golden table."""
    import pathlib
    rows = [l.split() for l in (pathlib.Path(__file__).parent / "golden" /
                                "e2m1_values.txt").read_text().splitlines()
            if l.strip() and not l.startswith("#")]
    return {int(c): Fraction(v) for c, v in rows}


def test_scores_fp4_query_bruteforce_exact():
    """The FP4-query score against exact rational arithmetic written from
    the format definitions alone: element 2i in the low nibble of byte i,
    sign bit 8, E8M0 scale byte g = 2**(g - 127) for elements 32g..32g+31."""
    mag = _e2m1_table()

    def deq(codes, scales):
        out = []
        for e in range(128):
            nib = (int(codes[e // 2]) >> (4 * (e % 2))) & 15
            v = mag[nib & 7] * (-1 if nib & 8 else 1)
            out.append(v * Fraction(2) ** (int(scales[e // 32]) - 127))
        return out

    rng = np.random.default_rng(11)
    for trial in range(3):
        qc, qs = O.pack_idx(rng.standard_normal((32, 128)).astype(np.float32)
                            * rng.uniform(0.01, 50))
        kc, ks = O.pack_idx(rng.standard_normal((5, 128)).astype(np.float32))
        w = rng.uniform(0, 1, 32).astype(np.float32)
        got = O.indexer_scores_fp4q(qc, qs, w, O.unpack_idx(kc, ks))
        qv = [deq(qc[h], qs[h]) for h in range(32)]
        for j in range(5):
            kv = deq(kc[j], ks[j])
            ref = Fraction(0)
            for h in range(32):
                dot = sum(a * b for a, b in zip(qv[h], kv))
                ref += Fraction(float(w[h])) * max(dot, Fraction(0))
            assert got[j] == pytest.approx(float(ref), rel=1e-14, abs=1e-300)


def test_scores_fp4_query_reduces_to_bf16_query():
    """A query already exact in MXFP4 (each 32-block: E2M1 values times one
    power of two, with a largest magnitude of 4 or 6 so the MX exponent
    rule returns that power) scores as the bf16-query path does."""
    rng = np.random.default_rng(12)
    vals = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    q = rng.choice(vals, size=(32, 4, 32)) * rng.choice([-1, 1], size=(32, 4, 32))
    q[..., 0] = rng.choice([4.0, 6.0], size=(32, 4))   # pins the block max
    q = q * np.exp2(rng.integers(-6, 6, size=(32, 4, 1)))
    q = q.reshape(32, 128).astype(np.float32)
    qc, qs = O.pack_idx(q)
    assert np.array_equal(O.unpack_idx(qc, qs), q.astype(np.float64))
    c = _case(40, 13)
    keys = O.unpack_idx(c["ic"], c["is_"])
    a = O.indexer_scores_fp4q(qc, qs, c["w"], keys)
    b = O.indexer_scores(_bf16(q), c["w"], keys)     # q is exact in bf16
    assert np.array_equal(a, b)


# --------------------------------------------------------------- top-k ----
def test_topk_bruteforce_and_ties():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 20, 300).astype(np.float64)      # many exact ties
    for k in (1, 7, 64, 300, 512):
        ranked = sorted(range(300), key=lambda j: (-s[j], j))[:k]
        want = sorted(ranked) + [-1] * max(0, k - 300)
        assert O.topk(s, k).tolist() == want


def test_topk_invariants():
    rng = np.random.default_rng(4)
    s = rng.standard_normal(5000)
    sel = O.topk(s, 512)
    assert np.all(np.diff(sel) > 0)
    mask = np.zeros(5000, bool)
    mask[sel] = True
    assert s[mask].min() >= s[~mask].max()


def test_topk_with_ids_reports_ids():
    s = np.array([1.0, 5.0, 5.0, 2.0])
    ids = np.array([40, 30, 10, 20])
    # 5.0 at ids 30 and 10 tie: lower id first; k = 2 -> {10, 30}
    assert O.topk(s, 2, ids=ids).tolist() == [10, 30]
    assert O.topk(s, 3, ids=ids).tolist() == [10, 20, 30]


def test_topk_gap():
    assert O.topk_gap([4.0, 3.0, 2.0], 2) == pytest.approx(1 / 3)
    assert O.topk_gap([4.0, 3.0], 2) == np.inf


# ----------------------------------------------------------- attention ----
def test_attention_vs_torch_sdpa():
    rng = np.random.default_rng(5)
    q = _bf16(rng.standard_normal((64, 512)))
    keys = rng.standard_normal((100, 512))
    got = O.mqa_decode(q, keys, SCALE)
    qt = torch.from_numpy(F.bf16_bits_to_f64(q))[None, :, None, :]
    kt = torch.from_numpy(keys)[None, None].expand(1, 64, 100, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, kt, scale=SCALE)[0, :, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attention_degenerate_cases():
    rng = np.random.default_rng(6)
    q = _bf16(rng.standard_normal((64, 512)))
    k1 = rng.standard_normal((1, 512))
    assert np.allclose(O.mqa_decode(q, k1, SCALE), np.repeat(k1, 64, 0))
    same = np.repeat(k1, 9, 0)
    assert np.allclose(O.mqa_decode(q, same, SCALE), np.repeat(k1, 64, 0))
    keys = rng.standard_normal((33, 512))
    o = O.mqa_decode(q, keys, SCALE)
    assert np.all(o <= keys.max(0) + 1e-12) and np.all(o >= keys.min(0) - 1e-12)


def test_attention_tiny_loops():
    rng = np.random.default_rng(7)
    q = _bf16(rng.standard_normal((64, 512)))
    keys = rng.standard_normal((5, 512))
    got = O.mqa_decode(q, keys, SCALE)
    qf = F.bf16_bits_to_f64(q)
    for h in (0, 17, 63):
        lg = [SCALE * math.fsum(qf[h, d] * keys[j, d] for d in range(512))
              for j in range(5)]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        z = math.fsum(e)
        for d in (0, 100, 511):
            want = math.fsum(e[j] / z * keys[j, d] for j in range(5))
            assert got[h, d] == pytest.approx(want, rel=1e-11, abs=1e-12)


# -------------------------------------------------------- whole layers ----
def test_sparse_equals_dense_when_k_covers_all():
    c = _case(40, 8)
    sel, out, _ = O.full_layer(c["mc"], c["ms"], c["ic"], c["is_"], 40,
                               c["qi"], c["w"], c["q"], c["sw"], 128, 512,
                               SCALE)
    assert sel[:40].tolist() == list(range(40)) and np.all(sel[40:] == -1)
    # dense attention over all entries + the window, by torch's routine
    keys = np.concatenate([O.unpack_main(c["mc"], c["ms"]),
                           O.unpack_swa(c["sw"])])
    qt = torch.from_numpy(F.bf16_bits_to_f64(c["q"]))[None, :, None, :]
    kt = torch.from_numpy(keys)[None, None].expand(1, 64, keys.shape[0], 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, kt, scale=SCALE)[0, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_reuse_with_full_topk_reproduces_full():
    c = _case(700, 9)
    sel, out, _ = O.full_layer(c["mc"], c["ms"], c["ic"], c["is_"], 700,
                               c["qi"], c["w"], c["q"], c["sw"], 128, 512,
                               SCALE)
    out2 = O.reuse_layer(c["mc"], c["ms"], sel, c["q"], c["sw"], 128, SCALE)
    assert np.array_equal(out, out2)


def test_full_layer_topk_is_bruteforce_over_scores():
    c = _case(900, 10)
    sel, _, sc = O.full_layer(c["mc"], c["ms"], c["ic"], c["is_"], 800,
                              c["qi"], c["w"], c["q"], c["sw"], 128, 512,
                              SCALE)
    assert len(sc) == 800                                    # causal bound
    order = sorted(range(800), key=lambda j: (-sc[j], j))[:512]
    assert sel.tolist() == sorted(order)


def test_hierarchical_equals_flat_when_pool_covers_all():
    c = _case(8 * 40 + 5, 11)
    n = c["n"]
    bk = O.block_keys(c["ic"], c["is_"], n)
    sel_h, out_h, pool, _ = O.hier_layer(
        c["mc"], c["ms"], c["ic"], c["is_"], bk, n, c["qi"], c["w"], c["q"],
        c["sw"], 128, 64, SCALE, n_keep=2048)
    assert pool[:n].tolist() == list(range(n)) and np.all(pool[n:] == -1)
    sel_f, out_f, _ = O.full_layer(c["mc"], c["ms"], c["ic"], c["is_"], n,
                                   c["qi"], c["w"], c["q"], c["sw"], 128, 64,
                                   SCALE)
    assert np.array_equal(sel_h, sel_f)
    assert np.allclose(out_h, out_f, rtol=0, atol=1e-12)


def test_hierarchical_stage2_is_fine_scoring_in_pool():
    c = _case(8 * 64, 12)
    n = c["n"]
    bk = O.block_keys(c["ic"], c["is_"], n)
    sel, _, pool, fine = O.hier_layer(
        c["mc"], c["ms"], c["ic"], c["is_"], bk, n, c["qi"], c["w"], c["q"],
        c["sw"], 128, 32, SCALE, n_keep=16)
    # pool = union of the 16 best blocks under block scores
    bs = O.indexer_scores(c["qi"], c["w"], F.bf16_bits_to_f64(bk))
    best = sorted(range(64), key=lambda b: (-bs[b], b))[:16]
    assert pool.tolist() == sorted(8 * b + i for b in best for i in range(8))
    # stage 2: brute-force fine scoring restricted to the pool
    keys = O.unpack_idx(c["ic"], c["is_"])
    allsc = O.indexer_scores(c["qi"], c["w"], keys)
    ranked = sorted(pool.tolist(), key=lambda j: (-allsc[j], j))[:32]
    assert sel.tolist() == sorted(ranked)


def test_attention_rows_with_far_apart_logits():
    # Heads whose logits sit thousands apart: each row needs its own maximum
    # subtracted, or the low rows underflow to 0/0.
    rng = np.random.default_rng(13)
    keys = rng.standard_normal((20, 512)) * 30.0
    qf = np.zeros((64, 512), np.float32)
    qf[0] = keys[3] * 3.0
    qf[1] = -keys[3] * 3.0
    qf[2:] = rng.standard_normal((62, 512))
    q = _bf16(qf)
    got = O.mqa_decode(q, keys, SCALE)
    assert np.all(np.isfinite(got))
    qt = torch.from_numpy(F.bf16_bits_to_f64(q))[None, :, None, :]
    kt = torch.from_numpy(keys)[None, None].expand(1, 64, 20, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, kt, scale=SCALE)[0, :, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-10)


# ------------------------------------- hierarchical decoder group (pages) --
def test_block_max_scores_bruteforce():
    rng = np.random.default_rng(21)
    sc = rng.standard_normal(101)
    for n, block in ((101, 8), (96, 8), (7, 8), (50, 4), (33, 1)):
        got = O.block_max_scores(sc, n, block)
        nb = -(-n // block)
        assert len(got) == nb
        for bi in range(nb):
            assert got[bi] == max(sc[j] for j in range(bi * block,
                                                       min(n, bi * block + block)))


def test_full_pool_bruteforce_with_ties():
    c = _case(203, 22)
    sel, out, pool, sc = O.full_pool_layer(
        c["mc"], c["ms"], c["ic"], c["is_"], 203, c["qi"], c["w"], c["q"],
        c["sw"], 128, 16, SCALE, n_keep=9, block=8)
    # brute force: blocks by (-max, block id), first 9, expanded below n
    bmax = [max(sc[j] for j in range(b * 8, min(203, b * 8 + 8)))
            for b in range(26)]
    order = sorted(range(26), key=lambda b: (-bmax[b], b))[:9]
    want = sorted(j for b in order for j in range(b * 8, b * 8 + 8) if j < 203)
    assert list(pool[:len(want)]) == want and np.all(pool[len(want):] == -1)
    # planted tie: two blocks with the same maximum at the cut -> lower block
    sc2 = np.zeros(40)
    sc2[[3, 12, 20, 35]] = [5.0, 4.0, 4.0, 1.0]    # blocks 0, 1, 2, 4
    p2 = O.hier_pool(O.block_max_scores(sc2, 40, 8), 40, 2, 8)
    assert list(p2) == list(range(0, 16))


def test_reindex_equals_full_when_pool_covers_all():
    c = _case(150, 23)
    sel_f, out_f, _ = O.full_layer(c["mc"], c["ms"], c["ic"], c["is_"], 150,
                                   c["qi"], c["w"], c["q"], c["sw"], 128, 32,
                                   SCALE)
    pool = np.concatenate([np.arange(150), -np.ones(10, np.int64)])
    sel_r, out_r, _ = O.reindex_layer(c["mc"], c["ms"], c["ic"], c["is_"],
                                      pool, c["qi"], c["w"], c["q"], c["sw"],
                                      128, 32, SCALE)
    assert np.array_equal(sel_f, sel_r)
    assert np.array_equal(out_f, out_r)


def test_reindex_with_full_query_keeps_full_topk():
    """Every block holding one of the Full layer's top-k has a block maximum
    >= the k-th score and every other block's maximum is below it, so with
    n_keep >= k the pool holds the whole top-k and a Reindex layer using
    the Full layer's own query reproduces it (no ties at the boundary)."""
    c = _case(3000, 24)
    sel, out, pool, sc = O.full_pool_layer(
        c["mc"], c["ms"], c["ic"], c["is_"], 3000, c["qi"], c["w"], c["q"],
        c["sw"], 128, 64, SCALE, n_keep=64, block=8)
    assert O.topk_gap(sc, 64) > 1e-9
    assert set(sel.tolist()) <= set(pool.tolist())
    sel_r, out_r, _ = O.reindex_layer(c["mc"], c["ms"], c["ic"], c["is_"],
                                      pool, c["qi"], c["w"], c["q"], c["sw"],
                                      128, 64, SCALE)
    assert np.array_equal(sel, sel_r)
    assert np.array_equal(out, out_r)


# ------------------------------------------- attention epilogue details --
def test_sink_limits_and_closed_form():
    c = _case(40, 31)
    keys = O.gather_keys(c["mc"], c["ms"], np.arange(40), c["sw"], 128)
    plain = O.mqa_decode(c["q"], keys, SCALE)
    # a sink at -inf changes nothing; a huge sink sends every weight to 0
    assert np.allclose(O.mqa_decode_sink(c["q"], keys, SCALE,
                                         np.full(64, -np.inf)), plain,
                       rtol=1e-13, atol=1e-13)
    assert np.abs(O.mqa_decode_sink(c["q"], keys, SCALE,
                                    np.full(64, 800.0))).max() < 1e-300
    # one key: a = e^l / (e^l + e^z), o = a k, for every head
    k1 = keys[:1]
    z = np.linspace(-3, 3, 64).astype(np.float32)
    q = F.bf16_bits_to_f64(c["q"])
    got = O.mqa_decode_sink(c["q"], k1, SCALE, z)
    for h in range(64):
        l = float(q[h] @ k1[0]) * SCALE
        a = math.exp(l) / (math.exp(l) + math.exp(float(z[h])))
        assert np.allclose(got[h], a * k1[0], rtol=1e-12, atol=1e-12)
    # no keys: the output is zero
    assert np.array_equal(O.mqa_decode_sink(c["q"], keys[:0], SCALE, z),
                          np.zeros((64, 512)))


def test_rope_derotate_hand_and_group_law():
    rng = np.random.default_rng(32)
    o = rng.standard_normal((3, 512))
    assert np.array_equal(O.rope_derotate(o, 0), o)          # t = 0
    got = O.rope_derotate(o, 5, theta=10000.0)
    assert np.array_equal(got[:, :448], o[:, :448])           # first 448 dims
    # pair 0 has frequency 1: rotation by -5 rad, by hand
    c, s = math.cos(-5.0), math.sin(-5.0)
    assert np.allclose(got[:, 448], o[:, 448] * c - o[:, 449] * s)
    assert np.allclose(got[:, 449], o[:, 448] * s + o[:, 449] * c)
    # pair i has frequency 10000^(-2i/64): pair 31 by hand
    w = 10000.0 ** (-62.0 / 64)
    c, s = math.cos(-5 * w), math.sin(-5 * w)
    assert np.allclose(got[:, 510], o[:, 510] * c - o[:, 511] * s)
    # pair norms are kept; R_{-t} R_{-u} = R_{-(t+u)} (with R_p = rotation by +p)
    n0 = o[:, 448::2] ** 2 + o[:, 449::2] ** 2
    n1 = got[:, 448::2] ** 2 + got[:, 449::2] ** 2
    assert np.allclose(n0, n1)
    assert np.allclose(O.rope_derotate(O.rope_derotate(o, 7), 11),
                       O.rope_derotate(o, 18), rtol=1e-12, atol=1e-12)


def test_derotated_output_is_relative():
    """The page's identity: with values stored rotated to their own position
    s (R_s e_s), R_{-t} o_t = sum_s a_s R_{s-t} e_s -- shifting every
    position by the same amount leaves the de-rotated output unchanged."""
    rng = np.random.default_rng(33)
    e = rng.standard_normal((6, 512))
    a = rng.dirichlet(np.ones(6))
    pos = np.array([3, 10, 11, 40, 41, 90])

    def rot(x, p):                      # R_p = de-rotation by -p
        return O.rope_derotate(x, -p)
    for shift in (0, 1000, 123457):
        o = sum(a[i] * rot(e[i:i + 1], pos[i] + shift) for i in range(6))
        d = O.rope_derotate(o, 95 + shift)
        if shift == 0:
            base = d
        assert np.allclose(d, base, rtol=1e-9, atol=1e-9)


# -------------------------------------------------------- compressor ----
def test_softmax_pool_bruteforce_and_limits():
    rng = np.random.default_rng(51)
    c = rng.standard_normal((3, 512))
    z = rng.standard_normal((3, 512)) * 3
    got = O.softmax_pool(c, z)
    for ch in range(0, 512, 37):
        ws = [math.exp(z[i, ch]) for i in range(3)]
        want = sum(ws[i] * c[i, ch] for i in range(3)) / sum(ws)
        assert got[ch] == pytest.approx(want, rel=1e-12, abs=1e-12)
    assert np.array_equal(O.softmax_pool(c[:1], z[:1]), c[0])       # m = 1
    assert np.allclose(O.softmax_pool(c, np.zeros_like(z)), c.mean(axis=0))
    zz = np.zeros_like(z)
    zz[2] = 1000.0                                                  # dominant
    assert np.allclose(O.softmax_pool(c, zz), c[2])


def test_compress_block_bruteforce():
    rng = np.random.default_rng(52)
    d, m = 16, 2
    hb = _bf16(rng.standard_normal((m, d)))
    wkv = _bf16(rng.standard_normal((512, d)) / 4)
    wz = _bf16(rng.standard_normal((512, d)) / 4)
    wik = _bf16(rng.standard_normal((128, 512)) / 16)
    c, cbar, ki = O.compress_block(hb, wkv, wz, wik)
    h, Wkv, Wz, Wik = (F.bf16_bits_to_f64(x) for x in (hb, wkv, wz, wik))
    for i in range(m):
        for o in (0, 7, 300, 511):
            assert c[i, o] == pytest.approx(
                math.fsum(h[i, j] * Wkv[o, j] for j in range(d)), rel=1e-13)
    zc = [[math.fsum(h[i, j] * Wz[o, j] for j in range(d)) for o in range(512)]
          for i in range(m)]
    for o in (3, 256):
        ws = [math.exp(zc[i][o]) for i in range(m)]
        want = sum(ws[i] * c[i, o] for i in range(m)) / sum(ws)
        assert cbar[o] == pytest.approx(want, rel=1e-12)
    for o in (0, 127):
        assert ki[o] == pytest.approx(
            math.fsum(cbar[j] * Wik[o, j] for j in range(512)), rel=1e-12)


def test_reuse_layer_ext_composition():
    """reuse_layer_ext (the reference of every sink / de-rotation GPU test)
    pinned by closed forms, not by its own formula: no sink and no position
    give reuse_layer exactly; position 0 gives the sink attention alone; one
    chosen key and no window give o_h = a_h R_{-t} k with
    a_h = e^l / (e^l + e^z), the rotation written out by hand for pairs 0
    and 31 at a non-default theta ("DeepSeek-V4: Towards Highly Efficient
    Million-Token Context Intelligence", other details: attention-sink and
    R_{-t} o_t equations)."""
    c = _case(30, 34)
    sel = np.array([3, 17, 29, -1, 8])
    base = O.reuse_layer(c["mc"], c["ms"], sel, c["q"], c["sw"], 100, SCALE)
    assert np.array_equal(
        O.reuse_layer_ext(c["mc"], c["ms"], sel, c["q"], c["sw"], 100, SCALE),
        base)
    z = np.linspace(-4, 4, 64).astype(np.float32)
    keys = O.gather_keys(c["mc"], c["ms"], sel, c["sw"], 100)
    assert np.array_equal(
        O.reuse_layer_ext(c["mc"], c["ms"], sel, c["q"], c["sw"], 100, SCALE,
                          sink=z, pos=0),
        O.mqa_decode_sink(c["q"], keys, SCALE, z))
    # One key, no window: closed form, head by head.
    t, theta = 77, 500.0
    got = O.reuse_layer_ext(c["mc"], c["ms"], np.array([12]), c["q"], c["sw"],
                            0, SCALE, sink=z, pos=t, theta=theta)
    k = O.unpack_main(c["mc"][12:13], c["ms"][12:13])[0]
    q = F.bf16_bits_to_f64(c["q"])
    for h in (0, 21, 63):
        l = math.fsum(float(q[h, d]) * float(k[d]) for d in range(512)) * SCALE
        a = math.exp(l) / (math.exp(l) + math.exp(float(z[h])))
        want = a * k.copy()
        for i in (0, 31):
            ang = -t * theta ** (-2.0 * i / 64)
            x, y = want[448 + 2 * i], want[449 + 2 * i]
            want[448 + 2 * i] = x * math.cos(ang) - y * math.sin(ang)
            want[449 + 2 * i] = x * math.sin(ang) + y * math.cos(ang)
        for d in (0, 200, 447, 448, 449, 510, 511):
            assert got[h, d] == pytest.approx(want[d], rel=1e-11, abs=1e-13)
    # A sink of -inf with a position is the plain attention, de-rotated.
    assert np.allclose(
        O.reuse_layer_ext(c["mc"], c["ms"], sel, c["q"], c["sw"], 100, SCALE,
                          sink=np.full(64, -np.inf), pos=t, theta=theta),
        O.rope_derotate(base, t, theta), rtol=1e-12, atol=1e-12)
