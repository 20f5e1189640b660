"""Pins of the oracle's cache packing: entry sizes the pages print, the
quantiser definition applied by exhaustive search in exact arithmetic,
PyTorch's independent E4M3/bf16 casts, and invariants of the OCP MX rule."""
import json
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import csa2 as O
from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]


def _gold(key):
    with open(os.path.join(GOLD, "page_figures.json")) as f:
        return json.load(f)[key]["value"]


def _nearest_e2m1(r):
    """Exhaustive nearest E2M1 magnitude to |r| (Fraction), ties to even
    code, saturating at 6; returns the signed value."""
    a = abs(r)
    best = min(range(8), key=lambda c: (abs(a - E2M1[c]), c & 1))
    return -E2M1[best] if r < 0 else E2M1[best]


def _rows(n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 512)) * scale).astype(np.float32)


def test_entry_sizes_match_pages():
    x = _rows(3, 0)
    c, s = O.pack_main(x)
    assert c.shape == (3, 256) and s.shape == (3, 32)
    assert c.shape[1] + s.shape[1] == _gold("main_entry_bytes")
    c2, s2 = O.pack_idx(x[:, :128])
    assert c2.shape[1] + s2.shape[1] == _gold("idx_entry_bytes")
    assert (c.shape[1] + s.shape[1] + c2.shape[1] + s2.shape[1]
            == _gold("entry_bytes"))


def test_main_scale_is_e4m3_of_amax_over_6():
    x = np.concatenate([_rows(64, 1), _rows(16, 2, 1e-3), _rows(16, 3, 300.0)])
    _, s = O.pack_main(x)
    amax = np.abs(x.reshape(-1, 32, 16)).max(-1)
    # torch's cast of the float32 quotient; the quotient's rounding cannot
    # move it across an E4M3 rounding boundary (see oracle/formats.py).
    ref = torch.from_numpy((amax / np.float32(6)).astype(np.float32))
    ref = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s, ref)


def test_main_codes_bruteforce_exact():
    x = np.concatenate([_rows(6, 4), _rows(2, 5, 1e-2), _rows(2, 6, 900.0)])
    codes, scales = O.pack_main(x)
    deq = O.unpack_main(codes, scales)
    for i in range(x.shape[0]):
        for g in range(32):
            s = Fraction(float(F.e4m3_decode(scales[i, g])))
            for j in range(16):
                ch = 16 * g + j
                xv = Fraction(float(x[i, ch]))
                want = _nearest_e2m1(xv / s) * s if s else Fraction(0)
                assert Fraction(float(deq[i, ch])) == want, (i, ch)


def test_main_nibble_order_and_layout():
    # A row built from known codes: group 0 scale 1.0 (amax 6 -> 6/6 = 1).
    x = np.zeros((1, 512), dtype=np.float32)
    x[0, 0] = 6.0      # code 7 in channel 0 (low nibble of byte 0)
    x[0, 1] = -0.5     # code 9 in channel 1 (high nibble of byte 0)
    x[0, 2] = 1.5      # code 3 (low nibble of byte 1)
    x[0, 17] = 3.0     # group 1: amax 3 -> scale E4M3(0.5); 3/0.5 = 6, code 7
    c, s = O.pack_main(x)
    assert c[0, 0] == 0x97 and c[0, 1] == 0x03
    assert c[0, 8] == 0x70                    # channel 17 is high nibble
    assert s[0, 0] == 0x38 and s[0, 1] == 0x30   # E4M3 1.0 and 0.5
    assert s[0, 2] == 0x00                    # all-zero group -> zero scale


def test_main_dynamic_range_2688():
    x = np.zeros((1, 512), dtype=np.float32)
    x[0, :16] = 2688.0
    x[0, 16:32] = -5000.0           # saturates at -448 * 6
    deq = O.unpack_main(*O.pack_main(x))
    assert np.all(deq[0, :16] == _gold("fp4_max_magnitude"))
    assert np.all(deq[0, 16:32] == -2688.0)


def test_main_roundtrip_error_bound():
    x = _rows(256, 7)
    codes, scales = O.pack_main(x)
    deq = O.unpack_main(codes, scales)
    s = F.e4m3_decode(scales).repeat(16, axis=1)
    r = np.abs(x.astype(np.float64)) / s
    err = np.abs(deq - x.astype(np.float64))
    # Half the E2M1 grid gap around |x|/s: 0.25 below 2, 0.5 below 4, 1 up
    # to 6; above 6 (scale rounded down) the value saturates to 6 s.
    bound = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, 1.0)) * s
    ok = r <= 6
    assert np.all(err[ok] <= bound[ok])
    assert np.all(np.abs(deq[~ok]) == 6 * s[~ok])


def test_signed_zero_and_zero_scale():
    x = np.zeros((1, 512), dtype=np.float32)
    x[0, 0] = -1e-9           # group 0: amax/6 far below 2**-10 -> scale 0
    x[0, 1] = 1e-9
    c, s = O.pack_main(x)
    assert s[0, 0] == 0 and c[0, 0] == 0x08   # -0 low nibble, +0 high


# ---------------------------------------------------------------- MXFP4 ---
def test_idx_scale_invariant_pins_exponent():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((500, 128)) *
         np.exp2(rng.integers(-20, 20, (500, 1)))).astype(np.float32)
    codes, scales = O.pack_idx(x)
    amax = np.abs(x.reshape(-1, 4, 32)).max(-1).astype(np.float64)
    sc = F.e8m0_decode(scales)
    # The OCP MX exponent is the unique integer e with 4 <= amax / 2**e < 8.
    r = amax / sc
    assert np.all((r >= 4) & (r < 8))


def test_idx_codes_bruteforce_exact():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    codes, scales = O.pack_idx(x)
    deq = O.unpack_idx(codes, scales)
    for i in range(8):
        for b in range(4):
            s = Fraction(float(F.e8m0_decode(scales[i, b])))
            for j in range(32):
                d = 32 * b + j
                want = _nearest_e2m1(Fraction(float(x[i, d])) / s) * s
                assert Fraction(float(deq[i, d])) == want


def test_idx_zero_block():
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 40] = 1.0
    c, s = O.pack_idx(x)
    assert s[0, 0] == 0 and s[0, 2] == 0 and s[0, 3] == 0
    assert s[0, 1] == 127 - 2            # amax 1 -> e = -2
    assert np.all(O.unpack_idx(c, s)[0, [i for i in range(128) if i != 40]]
                  == 0)
    assert O.unpack_idx(c, s)[0, 40] == 1.0


def test_swa_is_unscaled_e4m3():
    x = _rows(4, 10)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(O.pack_swa(x), ref.numpy())
    assert O.pack_swa(x).shape == (4, 512)


# ------------------------------------------------------------ block keys ---
def test_block_keys_bruteforce():
    rng = np.random.default_rng(11)
    n = 8 * 5 + 3                               # ragged last block of 3
    x = rng.standard_normal((n, 128)).astype(np.float32)
    c, s = O.pack_idx(x)
    bk = O.block_keys(c, s, n)
    assert bk.shape == (6, 128)
    deq = O.unpack_idx(c, s)
    for b in range(6):
        rows = range(8 * b, min(8 * b + 8, n))
        for d in range(0, 128, 7):
            mean = sum(Fraction(float(deq[r, d])) for r in rows) / len(rows)
            m32 = np.float32(float(mean))
            if Fraction(float(m32)) == mean:          # exactly representable
                ref = torch.tensor([m32]).to(torch.bfloat16).view(
                    torch.uint16).item()
                assert bk[b, d] == ref
            else:     # ragged block of 3: nearest bf16 to the exact mean
                got = F.bf16_bits_to_f64(bk[b, d])
                _, ex = np.frexp(got)
                half_ulp = Fraction(2) ** (int(ex) - 9)
                assert abs(Fraction(float(got)) - mean) <= half_ulp
