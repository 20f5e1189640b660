"""Oracle codecs: E2M1, E4M3 (OCP "FN"), E8M0 and bfloat16, written out from
their definitions in float64 NumPy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module;
only tests/, the smoke check and the CPU-baseline leg of the benchmark do.

Sources (web pages, cited by title):
  [KVC]  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
         (mer.run post), sections 2 and 5.
  [ARCH] "DeepSeek-V4.1-Flash, 2. Architecture" course notes
         (guaifinition.github.io), section 2.4.4 "FP4 main KV cache".

What the pages fix: main-KV values are E2M1 with one E4M3 scale per 16
channels and no global scale, the largest representable magnitude is
448 x 6 = 2688 ([ARCH] 2.4.4, [KVC] 5), and the indexer key is OCP MXFP4,
E2M1 with one E8M0 scale per 32 elements ([KVC] 2, [ARCH] 2.4.4).  The
pages do not state rounding or tie rules; the readings used here are:
round-to-nearest with ties to the even code, saturation at the largest
finite magnitude, and the sign of zero kept.

Exactness: every decision below is taken on the exact real value.  Inputs
are float32 (24-bit significands) and the divisors are E4M3 values (at most
4 significant bits) or powers of two, so the float64 quotient differs from
the exact one by at most 2**-53 relative, while a non-tied quotient sits at
least ~2**-27 relative away from any rounding threshold; float64 therefore
takes the same decision as exact arithmetic.
"""
import numpy as np

# ---------------------------------------------------------------- E2M1 ----
# 4-bit float: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN.
# Code c (low 3 bits) -> magnitude; c = (e << 1) | m.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def e2m1_decode(codes):
    """4-bit codes (0..15) -> float64 values; bit 3 is the sign."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_encode(r):
    """Round the real values r (float64, taken as exact) to E2M1 codes.

    Nearest representable magnitude, ties to the even code (mantissa bit 0),
    magnitudes above 6 saturate to 6.  The sign is kept, so a negative value
    that rounds to zero gives code 8 (negative zero).
    """
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    # The midpoints between consecutive magnitudes.
    mids = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0
    above = np.searchsorted(mids, a, side="left")   # midpoints below a
    tie = mids[np.minimum(above, len(mids) - 1)] == a
    code = np.where(tie & (above % 2 == 1), above + 1, above)
    sign = np.signbit(r).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------- E4M3 ----
# OCP FP8 E4M3 "FN": 1 sign, 4 exponent (bias 7), 3 mantissa bits.
# Exponent field 0 -> subnormal m/8 * 2**-6.  S.1111.111 is NaN; there is
# no infinity.  Largest finite magnitude 1.75 * 2**8 = 448.
E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANT_BITS = 3


def e4m3_decode(codes):
    """8-bit codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0,
                   m / 8.0 * 2.0 ** E4M3_MIN_NORMAL_EXP,
                   (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where((c & 0x80) != 0, -mag, mag)


def e4m3_encode(v):
    """Round real values v (float64, taken as exact) to E4M3 codes.

    Nearest representable value, ties to even mantissa, saturating at +-448
    (never producing the NaN codes).  The sign of zero is kept.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # Binade of a, clamped at the subnormal boundary: quantum = 2**(e-3).
    _, ex = np.frexp(np.where(a > 0, a, 1.0))       # a = f * 2**ex, f in [.5, 1)
    e = np.maximum(ex - 1, E4M3_MIN_NORMAL_EXP)
    quantum = np.exp2(e - E4M3_MANT_BITS)
    q = np.rint(a / quantum)                         # rint = ties-to-even
    val = np.minimum(q * quantum, E4M3_MAX)          # saturate
    # Re-derive the code from the rounded value (carries move up a binade).
    _, ex2 = np.frexp(np.where(val > 0, val, 1.0))
    e2 = ex2 - 1
    normal = val >= 2.0 ** E4M3_MIN_NORMAL_EXP
    mant_n = np.rint(val / np.exp2(e2) * 8.0 - 8.0)
    code_n = ((e2 + 7) << 3) + mant_n.astype(np.int64)
    code_s = np.rint(val / 2.0 ** (E4M3_MIN_NORMAL_EXP - E4M3_MANT_BITS))
    code = np.where(normal, code_n, code_s.astype(np.int64))
    code = np.where(val == 0, 0, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------- E8M0 ----
# OCP MX shared scale: 8-bit biased exponent, value 2**(c - 127); 255 = NaN.
def e8m0_decode(codes):
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


# ---------------------------------------------------------------- bf16 ----
def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(v):
    """Round real values (float64, taken as exact) to bfloat16, ties to even.

    Returns the uint16 bit patterns.  bfloat16 has 8 significant bits and
    float32's exponent range (subnormal quantum 2**-133).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -126)
    quantum = np.exp2(e - 7)
    val = np.rint(a / quantum) * quantum
    val = np.where(val > 3.3895313892515355e38, np.inf, val)   # past max+half ulp
    f32 = np.copysign(val, v).astype(np.float32)   # exact: val has <= 8 bits
    return (f32.view(np.uint32) >> 16).astype(np.uint16)
