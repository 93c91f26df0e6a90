"""Microscaled (MX) FP8 variant (test infrastructure only).

"The Insider Secrets Of Deepseek Discovered", passage after Figure 7: the
fine-grained scheme is consistent with microscaling formats, which the
next GPU generation supports with smaller groups.  The pages give no MX
definition, so the plainest reading is taken: the published OCP MX rule for
an MXFP8 (E4M3) block of 32 consecutive elements along the contraction axis,
with one shared power-of-two scale stored as an E8M0 byte:

    amax = max |x| over the block
    s    = floor(log2(amax)) - 8          (8 = exponent of E4M3's largest binade)
    s    = clamp(s, -127, 127)            (E8M0 range; amax = 0 gives -127)
    code = E4M3_RNE_SAT(RN32(x * 2^-s))   (|x| * 2^-s < 512; values past 448 saturate)
    byte = s + 127

So the scale only shifts exponents; unlike the method's amax / 448 scale the
largest element lands in [256, 512) and up to one binade of its group's
range saturates or goes unused.

Layouts: codes [R][K] row-major, scale bytes [K/32][R] (block-major, like the
1x128 scales).  GEMM: C = A . B^T with both operands MX-quantized along K.
"""

import numpy as np

from . import e4m3

BLOCK = 32
E4M3_EMAX = 8


def quant_mx_1x32(x):
    """x float32 [R][K] (K % 32 == 0) -> (codes u8 [R][K], scale bytes u8 [K/32][R])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    assert K % BLOCK == 0, "K must be a multiple of 32"
    t = x.reshape(R, K // BLOCK, BLOCK)
    amax = np.max(np.abs(t), axis=2).astype(np.float64)
    _, ex = np.frexp(amax)                    # amax = m * 2^ex, 0.5 <= m < 1
    s = np.where(amax > 0, ex - 1 - E4M3_EMAX, -127)
    s = np.clip(s, -127, 127).astype(np.int64)
    y = (t.astype(np.float64) * np.exp2(-s.astype(np.float64))[..., None]).astype(np.float32)
    q = e4m3.encode(y).reshape(R, K)
    return q, np.ascontiguousarray((s + 127).astype(np.uint8).T)


def scales_of(e):
    """E8M0 bytes -> float64 powers of two."""
    return np.exp2(np.asarray(e, dtype=np.float64) - 127.0)


def dequant_mx(q, e):
    """Exact float64 values of MX-quantized rows: q u8 [R][K], e u8 [K/32][R]."""
    return e4m3.decode(q) * np.repeat(scales_of(e).T, BLOCK, axis=1)


def quant_mx_1x32_transposed(x):
    """x float32 [M][K] (M % 32 == 0) -> (codes u8 [K][M], scale bytes u8 [M/32][K]):
    the same rule on blocks of 32 consecutive rows of one column, i.e. the
    rowwise quantizer applied to x^T.  These are the MX operands whose
    contraction runs over x's rows: X and dY of the Wgrad GEMM (tokens), and W
    of the Dgrad GEMM (output features)."""
    x = np.asarray(x, dtype=np.float32)
    return quant_mx_1x32(np.ascontiguousarray(x.T))
