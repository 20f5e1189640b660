"""Pins of the oracle codecs against things other than the oracle itself:
the format definitions applied by brute force in exact rational arithmetic,
PyTorch's independent float8/bfloat16 casts, and the figures the pages print.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLD, "page_figures.json")) as f:
        return json.load(f)


def _e2m1_table():
    vals = {}
    with open(os.path.join(GOLD, "e2m1_values.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals[int(c)] = float(v)
    return vals


# ---------------------------------------------------------------- E2M1 ----
def _e2m1_from_fields(code):
    """E2M1 value from its bit fields (sign, 2-bit exponent bias 1, 1-bit
    mantissa), independent of the oracle's table."""
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * 2 ** (e - 1)
    return -mag if s else mag


def test_e2m1_decode_table_exhaustive():
    gold = _e2m1_table()
    dec = F.e2m1_decode(np.arange(16))
    for c in range(16):
        assert dec[c] == float(_e2m1_from_fields(c))
        assert abs(dec[c]) == gold[c & 7]
        assert np.signbit(dec[c]) == bool(c & 8)


def test_fp4_range_matches_pages():
    g = _golden()
    assert F.E2M1_MAX == g["e2m1_max"]["value"]
    assert F.E4M3_MAX == g["e4m3_max"]["value"]
    assert F.E2M1_MAX * F.E4M3_MAX == g["fp4_max_magnitude"]["value"]
    assert max(abs(F.e2m1_decode(np.arange(16)))) == 6.0
    finite = F.e4m3_decode(np.arange(256))
    assert np.nanmax(np.abs(finite)) == 448.0


def _e2m1_brute(x):
    """Nearest E2M1 code to the rational x, ties to the even code, sign kept;
    exhaustive search over the 16 codes."""
    x = Fraction(x)
    best = None
    for c in range(16):
        v = _e2m1_from_fields(c)
        if (v < 0) != (x < 0) and v != 0:
            continue
        d = abs(x - v)
        key = (d, c & 1)          # smaller distance, then even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1] & 7
    neg = x < 0 or (x == 0 and str(float(x)).startswith("-"))
    return c | (8 if neg else 0)


def test_e2m1_encode_thresholds_and_ties():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    # Ties go to the even code: 0.25->0, .75->1.0, 1.25->1.0, 1.75->2,
    # 2.5->2, 3.5->4, 5->4.
    expect_val = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    for t, ev in zip(mids, expect_val):
        assert F.e2m1_decode(F.e2m1_encode(t)) == ev
        assert F.e2m1_decode(F.e2m1_encode(-t)) == -ev
        for y in (np.nextafter(t, 0.0), np.nextafter(t, 10.0)):
            assert F.e2m1_encode(y) == _e2m1_brute(Fraction(float(y)))
            assert F.e2m1_encode(-y) == _e2m1_brute(-Fraction(float(y)))
    # saturation and signed zero
    assert F.e2m1_encode(7.0) == 7 and F.e2m1_encode(1e30) == 7
    assert F.e2m1_encode(-1e30) == 15
    assert F.e2m1_encode(-0.0) == 8 and F.e2m1_encode(0.0) == 0
    assert F.e2m1_encode(-0.1) == 8


@settings(max_examples=400, deadline=None)
@given(st.floats(min_value=-20, max_value=20, allow_nan=False, width=32))
def test_e2m1_encode_random_vs_bruteforce(x):
    if x == 0:
        return
    assert F.e2m1_encode(x) == _e2m1_brute(Fraction(x))


# ---------------------------------------------------------------- E4M3 ----
def test_e4m3_decode_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    dec = F.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(dec), nan)
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(dec[~nan], ref[~nan])
    assert np.array_equal(np.signbit(dec[~nan]), np.signbit(ref[~nan]))


def _e4m3_finite_values():
    vals = F.e4m3_decode(np.arange(256))
    return [(c, Fraction(float(v))) for c, v in enumerate(vals)
            if not np.isnan(v) and not (v == 0 and c == 0x80)]


def _e4m3_brute(x):
    """Nearest finite E4M3 value to x (ties to even mantissa), saturating."""
    x = Fraction(x)
    x = max(min(x, Fraction(448)), Fraction(-448))
    best = None
    for c, v in _e4m3_finite_values():
        key = (abs(x - v), c & 1)
        if best is None or key < best[0]:
            best = (key, c, v)
    return best[2]


def _e4m3_midpoints():
    vals = sorted({float(v) for _, v in _e4m3_finite_values() if v >= 0})
    return [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]


def test_e4m3_encode_midpoints_vs_bruteforce():
    pts = []
    for m in _e4m3_midpoints():
        m32 = np.float32(m)
        assert float(m32) == m             # midpoints are exact in fp32
        pts += [m32, np.nextafter(m32, np.float32(0)),
                np.nextafter(m32, np.float32(1e9))]
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts])
    enc = F.e4m3_encode(pts.astype(np.float64))
    dec = F.e4m3_decode(enc)
    for x, d in zip(pts, dec):
        assert Fraction(float(d)) == _e4m3_brute(Fraction(float(x))), x


def test_e4m3_encode_vs_torch_cast():
    rng = np.random.default_rng(1)
    # log-uniform magnitudes over the whole E4M3 range incl. subnormals
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 200_000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    x = np.concatenate([x, np.float32(_e4m3_midpoints()),
                        -np.float32(_e4m3_midpoints())])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_saturation_and_zero():
    assert F.e4m3_encode(448.0) == 0x7E
    assert F.e4m3_encode(464.0) == 0x7E
    assert F.e4m3_encode(1e9) == 0x7E
    assert F.e4m3_encode(-1e9) == 0xFE
    assert F.e4m3_encode(0.0) == 0x00 and F.e4m3_encode(-0.0) == 0x80
    assert F.e4m3_encode(2.0 ** -10) == 0x00          # tie -> even (zero)
    assert F.e4m3_encode(np.nextafter(2.0 ** -10, 1)) == 0x01
    assert F.e4m3_encode(2.0 ** -9) == 0x01


# --------------------------------------------------------- E8M0 / bf16 ----
def test_e8m0_decode():
    d = F.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert d[0] == 2.0 ** -127 and d[1] == 2.0 ** -126
    assert d[2] == 0.5 and d[3] == 1.0 and d[4] == 2.0
    assert d[5] == 2.0 ** 127 and np.isnan(d[6])


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(100_000).astype(np.float32)
    x = np.concatenate([x, x * 1e-30, x * 1e30])
    # exact bf16 midpoints: bf16 values + half their ulp
    b = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    b = b[(b != 0) & (np.abs(b) > 2.0 ** -120) & (np.abs(b) < 2.0 ** 120)]
    _, ex = np.frexp(b.astype(np.float64))
    ulp = np.exp2(ex - 1 - 7.0)                      # 8 significant bits
    mid = (b.astype(np.float64) + np.sign(b) * ulp / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64),
                          b.astype(np.float64) + np.sign(b) * ulp / 2)
    x = np.concatenate([x, mid])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    got = F.bf16_round(x.astype(np.float64))
    assert np.array_equal(got.astype(np.uint16), ref.astype(np.uint16))
    back = F.bf16_bits_to_f64(got)
    assert np.array_equal(back,
                          torch.from_numpy(ref.view(np.int16)).view(
                              torch.bfloat16).to(torch.float64).numpy())
