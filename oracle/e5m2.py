"""E5M2 codec, written from the bit layout (test infrastructure only).

Used only by the format study (oracle/study.py): the method keeps E4M3 for
every tensor, and E5M2 is the format of the hybrid schemes it replaces
(DeepGEMM launch article (itstec.com.br), section "O que e FP8?", figure text
with E4M3 and E5M2; DeepSeek-V3 FP8 knowledge-base page (codingmall.com),
section on unified E4M3).

Format (OCP E5M2): 1 sign, 5 exponent bits with bias 15, 2 mantissa bits.
Exponent 0 holds subnormals m * 2^-16; exponent 31 holds +-inf (mantissa 0)
and NaN.  Largest finite magnitude 1.75 * 2^15 = 57344 (code 0x7B).
Encoding: nearest of the 124 finite non-negative magnitudes, ties to the code
whose mantissa LSB is 0, saturating at 57344, sign bit copied.
"""

import numpy as np

MAX_FINITE = 57344.0
CODE_MAX = 0x7B


def decode(codes):
    """Value of each E5M2 byte as float64 (exact); inf and NaN codes as such."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    exp = (c >> 2) & 0x1F
    man = c & 0x3
    sub = man * 2.0 ** -16
    nrm = (1.0 + man / 4.0) * np.exp2(exp.astype(np.float64) - 15.0)
    val = np.where(exp == 0, sub, nrm)
    val = np.where(exp == 31, np.where(man == 0, np.inf, np.nan), val)
    return np.where(sign == 1, -val, val)


MAGNITUDES = decode(np.arange(CODE_MAX + 1, dtype=np.uint8))
MIDPOINTS = (MAGNITUDES[:-1] + MAGNITUDES[1:]) / 2.0


def encode(y):
    """float32 values -> E5M2 codes: nearest, ties to even, saturate at 57344."""
    y32 = np.ascontiguousarray(y, dtype=np.float32)
    a = np.abs(y32).astype(np.float64)
    i = np.searchsorted(MIDPOINTS, a, side="left")
    i_clip = np.minimum(i, MIDPOINTS.size - 1)
    tie = (i < MIDPOINTS.size) & (MIDPOINTS[i_clip] == a)
    code = np.where(tie & (i % 2 == 1), i + 1, i)
    code = np.where(np.isnan(a), CODE_MAX, code)
    sign = np.signbit(y32).astype(np.int64)
    return (code | (sign << 7)).astype(np.uint8)
