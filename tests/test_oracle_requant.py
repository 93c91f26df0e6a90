"""Pins for the oracle's FP8 activation-cache requantization (CPU only).

The reference computation is rebuilt here in exact rational arithmetic
(Python Fractions): each step rounds explicitly to binary32 or to E4M3 by
searching the 127 finite magnitudes, so it shares no numpy float path with the
oracle.
"""
from fractions import Fraction

import numpy as np

from oracle import e4m3, quant


def _rn32(v):
    """Exact rational -> the nearest binary32 value (ties to even), gradual
    underflow; magnitudes stay far below the overflow threshold here."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    return r if v > 0 else -r


# E4M3FN finite magnitudes from the bit fields: exponent 0 -> m * 2^-9,
# otherwise (8 + m) * 2^(e - 10); codes 0..126
_MAGS = [Fraction(c & 7, 512) if c >> 3 == 0 else Fraction(8 + (c & 7)) * Fraction(2) ** ((c >> 3) - 10)
         for c in range(127)]


def _decode(code):
    """(negative?, exact magnitude) of a non-NaN code."""
    return bool(code & 0x80), _MAGS[code & 0x7F]


def _encode(neg, mag):
    """Round-to-nearest-even, saturating at 448; the sign bit is kept."""
    if mag >= 448:
        best = 0x7E
    else:
        best = None
        for c, m in enumerate(_MAGS):
            d = abs(m - mag)
            if best is None or d < bd or (d == bd and c % 2 == 0):
                best, bd = c, d
    return (0x80 if neg else 0) | best


def _brute_requant(q, s):
    R, K = q.shape
    # x' = RN32(dec * s), with its sign bit (s >= 0; -0 codes stay -0)
    xs = [[None] * K for _ in range(R)]
    for r in range(R):
        for k in range(K):
            neg, mag = _decode(int(q[r, k]))
            xs[r][k] = (neg, _rn32(mag * Fraction(float(s[k // 128, r]))))
    qt = np.zeros((K, R), np.uint8)
    st = np.zeros((R // 128, K), np.float32)
    for k in range(K):
        for tb in range(R // 128):
            tile = [xs[tb * 128 + i][k] for i in range(128)]
            amax = max(m for _, m in tile)
            sc = _rn32(amax / 448)
            st[tb, k] = np.float32(float(sc))
            for i, (neg, m) in enumerate(tile):
                y = m if sc == 0 else _rn32(m / sc)
                qt[k, tb * 128 + i] = _encode(neg, y)
    return qt, st


def _random_cache(rng, R, K):
    q = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E                    # no NaN codes in a cache
    s = np.exp(rng.uniform(np.log(1e-6), np.log(1e3), size=(K // 128, R))).astype(np.float32)
    s[0, 5] = 0.0                                   # a zero row scale
    s[0, 6] = np.float32(3e-40)                     # a subnormal row scale
    s[1, 7] = np.float32(2.0 ** -20)                # a power of two
    q[9, :] = 0x80                                  # a row of -0 codes
    return q, s


def test_requant_matches_exact_rational_brute_force():
    rng = np.random.default_rng(2024)
    q, s = _random_cache(rng, 128, 256)
    # one channel whose whole token tile dequantizes to zeros of both signs
    q[:, 3] = np.where(np.arange(128) % 2 == 0, 0x00, 0x80)
    qt, st = quant.requant_act_tokenwise(q, s)
    bq, bs = _brute_requant(q, s)
    assert np.array_equal(st.view(np.uint32), bs.view(np.uint32))
    bad = np.argwhere(qt != bq)
    assert bad.size == 0, bad[:5].tolist()
    assert st[0, 3] == 0.0 and np.array_equal(qt[3], q[:, 3])


def test_power_of_two_row_scales_make_the_dequantization_exact():
    """With power-of-two row scales dec(q) * s is exact in float32, so the
    requantization is the token-wise quantization of the exact values."""
    rng = np.random.default_rng(7)
    R, K = 256, 384
    q = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x00
    s = (2.0 ** rng.integers(-30, 10, size=(K // 128, R))).astype(np.float32)
    exact = quant.dequant_act(q, s)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    qt, st = quant.requant_act_tokenwise(q, s)
    eq, es = quant.quant_act_1x128_tokenwise(exact.astype(np.float32))
    assert np.array_equal(qt, eq) and np.array_equal(st.view(np.uint32), es.view(np.uint32))


def test_requant_error_against_the_cached_values():
    """Each requantized value lies within half an E4M3 step (of y = x'/st) of
    the dequantized cache value x', plus the division's float32 slack."""
    rng = np.random.default_rng(11)
    q, s = _random_cache(rng, 256, 256)
    xq = quant.dequant32(q, np.repeat(s.T, 128, axis=1)).astype(np.float64)      # [R][K]
    qt, st = quant.requant_act_tokenwise(q, s)
    st_full = np.repeat(st, 128, axis=0).astype(np.float64)                          # [R][K]
    back = e4m3.decode(qt).T * st_full
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(st_full > 0, np.abs(xq) / st_full, 0.0)
    ulp = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(y, 2.0 ** -30))), -6) - 3)
    lim = (ulp / 2 + 2.0 ** -23 * y) * st_full
    assert np.all(np.abs(back - xq) <= lim)
