"""E4M3 codec, written from the bit layout (test infrastructure only).

Format: DeepGEMM launch article (itstec.com.br), section "O que e FP8?" -- the
figure text gives E4M3 as 4 exponent bits and 3 mantissa bits beside E5M2.
Flavour (reading): OCP E4M3FN -- exponent bias 7, no infinities, the two codes
with all exponent and mantissa bits set (0x7F, 0xFF) are NaN, so the largest
finite magnitude is 1.75 * 2^8 = 448.

Decoding is the closed form of the bit fields.  Encoding is the plain
definition of round-to-nearest-even with saturation: the nearest of the 127
finite non-negative magnitudes, ties going to the code whose mantissa LSB is
0, magnitudes beyond 448 clamped to 448, sign bit copied from the input (so
-0 and small negatives that round to zero give 0x80).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MAX_FINITE = 448.0
CODE_MAX = 0x7E          # +448
NAN_CODES = (0x7F, 0xFF)


def decode(codes):
    """Value of each E4M3 byte as float64 (exact).  NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man * 2.0 ** -9                                   # exp == 0: 0.mmm * 2^(1-7)
    nrm = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    val = np.where(exp == 0, sub, nrm)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return np.where(sign == 1, -val, val)


# The 127 finite non-negative magnitudes, indexed by their code (0x00..0x7E);
# decode() is monotone in the code over this range.
MAGNITUDES = decode(np.arange(CODE_MAX + 1, dtype=np.uint8))
# Halfway points between neighbouring magnitudes (exact in float64).
MIDPOINTS = (MAGNITUDES[:-1] + MAGNITUDES[1:]) / 2.0


_CHUNK = 1 << 20


def _threads():
    n = os.environ.get("OMP_NUM_THREADS")
    try:
        n = int(n) if n else len(os.sched_getaffinity(0))
    except (ValueError, AttributeError):
        n = os.cpu_count() or 1
    return max(1, min(n, 32))


def encode(y):
    """Round float32 values to E4M3 codes: nearest, ties to even, saturate at 448.

    ``y`` is taken as float32 (the method scales in float32 before casting).
    Non-finite input is outside the contract: NaN and +-inf both come out as
    the saturated code.  Large arrays are split into independent chunks that
    are encoded on a thread pool (each element is computed the same way).
    """
    y32 = np.ascontiguousarray(y, dtype=np.float32)
    if y32.size <= 2 * _CHUNK:
        return _encode_flat(y32)
    flat = y32.reshape(-1)
    out = np.empty(flat.shape, np.uint8)

    def job(start):
        out[start:start + _CHUNK] = _encode_flat(flat[start:start + _CHUNK])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(0, flat.size, _CHUNK)))
    return out.reshape(y32.shape)


def _encode_flat(y32):
    a = np.abs(y32).astype(np.float64)
    # i = number of midpoints strictly below |y|: the nearest magnitude's code
    # unless |y| sits exactly on midpoint i (a tie between codes i and i+1).
    i = np.searchsorted(MIDPOINTS, a, side="left")
    i_clip = np.minimum(i, MIDPOINTS.size - 1)
    tie = (i < MIDPOINTS.size) & (MIDPOINTS[i_clip] == a)
    code = np.where(tie & (i % 2 == 1), i + 1, i)            # even code wins a tie
    code = np.where(np.isnan(a), CODE_MAX, code)
    sign = np.signbit(y32).astype(np.int64)
    return (code | (sign << 7)).astype(np.uint8)


def ulp_at(y):
    """Spacing of E4M3 values around |y| (float64): 2^(max(floor(log2|y|), -6) - 3)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, e, -6.0)
    return np.exp2(np.maximum(e, -6.0) - 3.0)
