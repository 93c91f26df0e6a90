"""Pins for the oracle's E4M3 codec (CPU only).

Independent references used here: the closed form of the bit layout, hand-worked
cases in tests/golden/, and PyTorch's own float8_e4m3fn cast (a library
routine that shares nothing with the oracle), which rounds to nearest-even and
agrees with a saturating cast for every |y| <= 464.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3
from tests.goldens import e4m3_cases


def torch_encode(y32):
    return torch.from_numpy(np.ascontiguousarray(y32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_code_table_closed_form():
    v = e4m3.decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2
    pos = v[:0x7F]
    assert pos.size == 127 and np.all(np.diff(pos) > 0)
    assert pos[0] == 0.0 and pos[1] == 2.0 ** -9 and pos[7] == 7 * 2.0 ** -9
    assert pos[8] == 2.0 ** -6 and pos[0x7E] == 448.0 and pos[0x7D] == 416.0
    # negative half mirrors the positive half, including -0
    assert np.all(v[0x80:0xFF] == -pos)
    assert np.signbit(v[0x80])


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(ours[ok]))


def test_golden_hand_cases():
    for val, code in e4m3_cases():
        got = int(e4m3.encode(np.float32(val)))
        assert got == code, (val, hex(got), hex(code))


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    y = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(y), codes)


def _binade(e):
    """All positive fp32 values with unbiased exponent e."""
    base = np.uint32((e + 127) << 23)
    return (np.arange(1 << 23, dtype=np.uint32) + base).view(np.float32)


@pytest.mark.parametrize("e", list(range(-11, 9)))
def test_exhaustive_binade_against_torch(e):
    """Every fp32 with exponent in [-11, 8] (covers 2^-11 .. 512): positive and
    negative values must encode exactly as the library cast, except that
    magnitudes above 464 (where the library returns NaN) saturate to 448."""
    y = _binade(e)
    ours = e4m3.encode(y)
    lib = torch_encode(y)
    big = np.abs(y) > 464.0
    assert np.array_equal(ours[~big], lib[~big])
    assert np.all(ours[big] == 0x7E)
    neg = -y[::97]
    assert np.array_equal(e4m3.encode(neg)[np.abs(neg) <= 464], torch_encode(neg)[np.abs(neg) <= 464])


def test_tiny_and_huge_values():
    rng = np.random.default_rng(0)
    tiny = (rng.integers(0, 0x3A000000, size=1 << 20, dtype=np.uint32)).view(np.float32)  # < 2^-11
    assert np.all(e4m3.encode(tiny) == 0)
    assert np.all(e4m3.encode(-tiny) == 0x80)
    huge = np.float32(2.0) ** rng.uniform(9, 127, size=4096).astype(np.float32)
    assert np.all(e4m3.encode(huge) == 0x7E) and np.all(e4m3.encode(-huge) == 0xFE)


def test_half_ulp_bound_and_monotone():
    rng = np.random.default_rng(1)
    y = np.sort(rng.uniform(0, 448, size=1 << 20).astype(np.float32))
    q = e4m3.encode(y)
    err = np.abs(e4m3.decode(q) - y.astype(np.float64))
    assert np.all(err <= e4m3.ulp_at(y) / 2)
    assert np.all(np.diff(q.astype(np.int64)) >= 0)


def test_ulp_at_is_the_code_spacing():
    """ulp_at(|y|) is the distance from E4M3 value dec(c) to the next one,
    dec(c + 1), for every code 0x00..0x7D (the subnormal step 2^-9 below 2^-6,
    2^(e-3) in binade e), and the same anywhere strictly between the two."""
    codes = np.arange(0x7E, dtype=np.uint8)
    lo = e4m3.decode(codes)
    hi = e4m3.decode(codes + 1)
    step = hi - lo
    assert np.array_equal(e4m3.ulp_at(lo), step)
    assert np.array_equal(e4m3.ulp_at((lo + hi) / 2.0), step)
    assert np.array_equal(e4m3.ulp_at(-lo), step)
    # closed forms at the edges of the range
    assert e4m3.ulp_at(0.0) == 2.0 ** -9
    assert e4m3.ulp_at(2.0 ** -9) == 2.0 ** -9
    assert e4m3.ulp_at(2.0 ** -6) == 2.0 ** -9          # first normal binade keeps the subnormal step
    assert e4m3.ulp_at(2.0 ** -5) == 2.0 ** -8
    assert e4m3.ulp_at(255.0) == 16.0 and e4m3.ulp_at(256.0) == 32.0 and e4m3.ulp_at(448.0) == 32.0
