"""Exact rational reimplementation of one quantization group (test helper).

Each step rounds explicitly: binary32 by round-to-nearest-even on the exact
rational, E4M3 by searching the 127 finite magnitudes.  Shares no code path
with the oracle's numpy arithmetic."""
from fractions import Fraction

import numpy as np

MAGS = [Fraction(c & 7, 512) if c >> 3 == 0 else Fraction(8 + (c & 7)) * Fraction(2) ** ((c >> 3) - 10)
        for c in range(127)]


def rn32(v):
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * ulp if v > 0 else -fl * ulp


def e4m3_rne(neg, mag):
    if mag >= 448:
        c = 0x7E
    else:
        c, bd = None, None
        for k, m in enumerate(MAGS):
            d = abs(m - mag)
            if c is None or d < bd or (d == bd and k % 2 == 0):
                c, bd = k, d
    return (0x80 if neg else 0) | c


def quant_group(vals):
    """vals: float32 values of one group -> (scale as float32, list of codes)."""
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fr)
    s = rn32(amax / 448)
    codes = []
    for v, f in zip(vals, fr):
        neg = bool(np.signbit(v))
        y = abs(f) if s == 0 else abs(rn32(f / s))
        codes.append(e4m3_rne(neg, y))
    return np.float32(float(s)), codes


# E5M2 (OCP): 1 sign, 5 exponent bits with bias 15, 2 mantissa bits; exponent 0
# holds the subnormals m * 2^-16; exponent 31 is inf / NaN, so the 124 finite
# non-negative magnitudes are codes 0x00..0x7B, the largest (4 + 3) * 2^13.
MAGS_E5M2 = [Fraction(c & 3, 1 << 16) if c >> 2 == 0 else Fraction(4 + (c & 3)) * Fraction(2) ** ((c >> 2) - 17)
             for c in range(124)]


def rne_to_grid(mag, mags):
    """Nearest of the non-negative magnitudes `mags` (ascending, code = index),
    ties to the even code, saturating at the largest: the code."""
    if mag >= mags[-1]:
        return len(mags) - 1
    c, bd = None, None
    for k, m in enumerate(mags):
        d = abs(m - mag)
        if c is None or d < bd or (d == bd and k % 2 == 0):
            c, bd = k, d
    return c


def quant_dequant_group(vals, mags):
    """One group quantized and dequantized exactly as the method does it, in the
    format whose magnitudes are `mags`: s = RN32(amax / max), y = RN32(x / s),
    code = RNE(y); returns the exact dequantized values dec(code) * s."""
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fr)
    s = rn32(amax / mags[-1])
    out = []
    for v, f in zip(vals, fr):
        if s == 0:
            out.append(Fraction(0))
            continue
        y = rn32(f / s)
        m = mags[rne_to_grid(abs(y), mags)]
        out.append((m if y >= 0 else -m) * s)
    return out
