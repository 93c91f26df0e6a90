"""Accumulation emulators for the limited-precision demonstration (test infrastructure only).

"The Insider Secrets Of Deepseek Discovered" reports that FP8 GEMM on H800
Tensor Cores keeps only about 14 bits while accumulating, that this led to a
maximum relative error of nearly 2% at an inner dimension of 4096 in a
preliminary test, and that the error grows with the inner dimension (passage
citing Wortsman et al.).  The remedy (passage on Figure 7(b)) promotes partial
results to FP32 registers at a fixed interval and applies the scales there;
the interval is garbled on that page and is read as 128, one K-block.

Emulators (all vectorised over the outputs, looping over k in order):
  * accum_limited       -- running sum rounded to `bits` significant bits after
                           every addition, no promotion (RN-even or toward zero).
  * accum_fp32_promoted -- the method: each 128-wide K-block summed in FP32
                           from exact code products, then acc += P * (sA * sB)
                           in FP32.
The exact value is oracle.gemm.gemm_ref.
"""

import numpy as np

from . import e4m3


def round_sig(v, bits, mode="rn"):
    """Round float64 values to `bits` significant bits (mode 'rn' = nearest-even, 'rz' = toward zero)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, bits)
    r = np.rint(scaled) if mode == "rn" else np.trunc(scaled)
    return np.ldexp(r, e - bits)


def accum_limited(a_dq, b_dq, bits=14, mode="rn"):
    """C[m,n] = sum_k a[m,k] b[n,k] with the running sum held to `bits` significant bits."""
    a = np.asarray(a_dq, dtype=np.float64)
    b = np.asarray(b_dq, dtype=np.float64)
    acc = np.zeros((a.shape[0], b.shape[0]))
    for k in range(a.shape[1]):
        acc = round_sig(acc + np.outer(a[:, k], b[:, k]), bits, mode)
    return acc


def accum_fp32_promoted(qa, sa, qb, sb, bscale_kind="128x128"):
    """The method's accumulation, emulated in float32.

    qa u8 [M][K], sa f32 [K/128][M]; qb u8 [N][K], sb f32 [N/128][K/128]
    ('128x128') or [K/128][N] ('1x128').  Per K-block kb:
        P   = sum_{k in kb} dec(qa[m,k]) * dec(qb[n,k])     float32, k in order
        acc = RN32(acc + RN32(P * RN32(sA[kb,m] * sB[.,kb])))
    Products of two E4M3 values have at most 8 significant bits, so each is
    exact in float32.
    """
    da = e4m3.decode(qa).astype(np.float32)
    db = e4m3.decode(qb).astype(np.float32)
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    M, K = da.shape
    N = db.shape[0]
    acc = np.zeros((M, N), dtype=np.float32)
    for kb in range(K // 128):
        p = np.zeros((M, N), dtype=np.float32)
        for k in range(kb * 128, kb * 128 + 128):
            p = (p + np.outer(da[:, k], db[:, k]).astype(np.float32)).astype(np.float32)
        if bscale_kind == "128x128":
            sbk = np.repeat(sb[:, kb], 128)[None, :]          # per column n: sB[n/128][kb]
        else:
            sbk = sb[kb][None, :]
        s = (sa[kb][:, None] * sbk).astype(np.float32)
        acc = (acc + (p * s).astype(np.float32)).astype(np.float32)
    return acc
