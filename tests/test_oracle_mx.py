"""Pins for the oracle's MX (1x32, E8M0 scale) quantizer (CPU only)."""
from fractions import Fraction

import numpy as np

from oracle import e4m3, mx

# E4M3 finite magnitudes from the bit fields (codes 0..126), as exact rationals
_MAGS = [Fraction(c & 7, 512) if c >> 3 == 0 else Fraction(8 + (c & 7)) * Fraction(2) ** ((c >> 3) - 10)
         for c in range(127)]


def _floor_log2(a):
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _rne_e4m3(neg, mag):
    if mag >= 448:
        c = 0x7E
    else:
        c, bd = None, None
        for k, m in enumerate(_MAGS):
            d = abs(m - mag)
            if c is None or d < bd or (d == bd and k % 2 == 0):
                c, bd = k, d
    return (0x80 if neg else 0) | c


def _brute(x):
    """The MX rule in exact rational arithmetic.  x * 2^-s is exact in binary32
    for the inputs used here (no fp32 underflow), so no rounding step is needed
    before the E4M3 rounding."""
    R, K = x.shape
    q = np.zeros((R, K), np.uint8)
    e = np.zeros((K // 32, R), np.uint8)
    for r in range(R):
        for b in range(K // 32):
            vals = [Fraction(float(v)) for v in x[r, 32 * b:32 * b + 32]]
            amax = max(abs(v) for v in vals)
            s = -127 if amax == 0 else max(-127, min(127, _floor_log2(amax) - 8))
            e[b, r] = s + 127
            for i, v in enumerate(vals):
                neg = bool(np.signbit(x[r, 32 * b + i]))
                q[r, 32 * b + i] = _rne_e4m3(neg, abs(v) / Fraction(2) ** s)
    return q, e


def test_matches_exact_rational_brute_force():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((6, 128)) * np.exp(rng.uniform(-8, 8, size=(6, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 5] = -0.0
    x[1, 32:64] = np.float32(1.9)                # saturates: 1.9 * 2^8 = 486.4 -> 448
    x[2, 64:96] = np.float32(2.0 ** -20) * np.arange(32, dtype=np.float32)
    q, e = mx.quant_mx_1x32(x)
    bq, be = _brute(x)
    assert np.array_equal(e, be)
    assert np.array_equal(q, bq)


def test_worked_blocks():
    """Hand-worked: a block whose amax is 1.0 gets s = -8 (byte 119), so the
    elements are scaled by 256; 1.9 saturates; a zero block keeps byte 0."""
    x = np.zeros((1, 96), np.float32)
    x[0, 0] = 1.0                                 # -> 256 = 1.0 * 2^8: code 0x78 (exp 15, mantissa 0)
    x[0, 1] = -0.5                                # -> -128: code 0xF0
    x[0, 2] = 1.0 / 256                           # -> 1.0: code 0x38
    x[0, 32] = 1.9                                # block 1: s = -8, 486.4 saturates to 448 = 0x7E
    x[0, 33] = 1.0                                # -> 256 = 0x78
    q, e = mx.quant_mx_1x32(x)
    assert e[:, 0].tolist() == [119, 119, 0]
    assert q[0, :3].tolist() == [0x78, 0xF0, 0x38]
    assert q[0, 32] == 0x7E and q[0, 33] == 0x78
    assert np.all(q[0, 64:] == 0)
    assert e4m3.decode(np.uint8(0x78)) == 256.0


def test_scale_range_and_power_of_two_equivariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    q, e = mx.quant_mx_1x32(x)
    for k in (-20, -3, 5, 30):
        q2, e2 = mx.quant_mx_1x32((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(q2, q) and np.array_equal(e2.astype(int), e.astype(int) + k)
    # the largest element of every block lands in [256, 448] after scaling
    big = np.abs(e4m3.decode(q)).reshape(8, 2, 32).max(axis=2)
    assert np.all((big >= 256) & (big <= 448))


def test_dequant_error_bound():
    """|dec * 2^s - x| <= half an E4M3 step of x * 2^-s, or the saturation
    loss for elements past 448 * 2^s."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((64, 256)) * 10).astype(np.float32)
    q, e = mx.quant_mx_1x32(x)
    back = mx.dequant_mx(q, e)
    scale = np.repeat(mx.scales_of(e).T, 32, axis=1)
    y = np.abs(x.astype(np.float64)) / scale
    lim = np.where(y > 448, y - 448 + 1e-12, e4m3.ulp_at(y) / 2) * scale
    assert np.all(np.abs(back - x) <= lim * (1 + 1e-12))


def test_transposed_blocks_run_down_the_columns():
    """The transposed quantizer's blocks are 32 consecutive rows of one column:
    against the exact brute force on x^T, and a column whose 32-row blocks have
    maxima 2^j (j = 0, 1, 2) gets scale bytes 127 + j - 8 in rows j of e."""
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((96, 5)) * np.exp(rng.uniform(-4, 4, size=(1, 5)))).astype(np.float32)
    q, e = mx.quant_mx_1x32_transposed(x)
    bq, be = _brute(np.ascontiguousarray(x.T))
    assert q.shape == (5, 96) and e.shape == (3, 5)
    assert np.array_equal(q, bq) and np.array_equal(e, be)
    y = np.full((96, 2), 0.25, np.float32)
    for j in range(3):
        y[32 * j + 7, 0] = np.float32(2.0 ** j)
    _, ey = mx.quant_mx_1x32_transposed(y)
    assert ey[:, 0].tolist() == [119, 120, 121]
    assert ey[:, 1].tolist() == [117, 117, 117]          # amax 2^-2: s = -2 - 8
