"""Reference for the block-scaled FP8 GEMMs (test infrastructure only).

The GEMM formula itself is lost from the DeepGEMM launch article ("O que e
Gemm?" ends before it); reading: C = A . B^T with both operands stored K-major
(rows of A and rows of B run along the contraction), no alpha/beta, no bias.
That is y = x . W^T for a Linear layer with W [out][in].

What the kernels compute ("The Insider Secrets Of Deepseek Discovered",
passages on limited Tensor Core accumulation and on promotion, Figure 7(b)):
each 128-wide K-block is accumulated on its own and then promoted into an
FP32 accumulator, the product of the two group scales being applied at that
promotion.  Up to rounding that equals the plain product of the dequantized
operands, which is what this module computes, exactly: every dequantized value
dec(q) * s has at most 4 + 24 significant bits and is exact in float64, and a
float64 dot product of length K carries an error below K * 2^-53 * S.

The GPU result is accepted when, element by element,
    FP32 output:  |C - C_ref| <= u * S
    BF16 output:  |C - C_ref| <= u * S * (1 + 2^-8) + 2^-8 * |C_ref|
with u = 2^-14 and S = sum_k |a_k b_k| over the dequantized operands.  The BF16
form adds one round-to-nearest to 8 significant bits of the FP32 accumulator
(relative error at most 2^-8) on top of the FP32 bound.
"""

import numpy as np

from . import quant

U = 2.0 ** -14
BF16_UNIT = 2.0 ** -8


def gemm_ref(a_dq, b_dq):
    """C_ref = A . B^T and S = |A| . |B|^T in float64 (a_dq [M][K], b_dq [N][K])."""
    a = np.asarray(a_dq, dtype=np.float64)
    b = np.asarray(b_dq, dtype=np.float64)
    return a @ b.T, np.abs(a) @ np.abs(b).T


def bound(c_ref, s_abs, out_dtype):
    """Element-wise acceptance bound for a GPU result (out_dtype 'bf16' or 'fp32')."""
    if out_dtype == "fp32":
        return U * s_abs
    if out_dtype == "bf16":
        return U * s_abs * (1.0 + BF16_UNIT) + BF16_UNIT * np.abs(c_ref)
    raise ValueError(out_dtype)


def b_dequant(qb, sb, bscale_kind):
    """Dequantize the B operand: '128x128' (sb [N/128][K/128]) or '1x128' (sb [K/128][N])."""
    if bscale_kind == "128x128":
        return quant.dequant_weight(qb, sb)
    if bscale_kind == "1x128":
        return quant.dequant_act(qb, sb)
    raise ValueError(bscale_kind)


def gemm_blockscaled_ref(qa, sa, qb, sb, bscale_kind="128x128", rows=None):
    """Dense block-scaled GEMM reference.

    qa u8 [M][K], sa f32 [K/128][M]; qb u8 [N][K] with sb as ``bscale_kind``.
    ``rows`` (optional index array) restricts the check to sampled rows of C.
    Returns (C_ref, S) for those rows.
    """
    qa = np.asarray(qa)
    sa = np.asarray(sa, dtype=np.float32)
    if rows is not None:
        rows = np.asarray(rows)
        qa = qa[rows]
        sa = sa[:, rows]
    return gemm_ref(quant.dequant_act(qa, sa), b_dequant(qb, sb, bscale_kind))


def grouped_contiguous_ref(qa, sa, qb, sb, group_offsets, rows=None):
    """Contiguous MoE layout: rows [off[g], off[g+1]) of A belong to expert g.

    qa u8 [M_total][K], sa [K/128][M_total], qb u8 [G][N][K], sb [G][N/128][K/128].
    Returns (row_index, C_ref, S) for the checked rows (all rows by default).
    """
    off = np.asarray(group_offsets, dtype=np.int64)
    m_total = qa.shape[0]
    rows = np.arange(m_total) if rows is None else np.sort(np.asarray(rows))
    out_c, out_s = [], []
    for g in range(off.size - 1):
        sel = rows[(rows >= off[g]) & (rows < off[g + 1])]
        if sel.size == 0:
            continue
        c, s = gemm_blockscaled_ref(qa, sa, qb[g], sb[g], "128x128", rows=sel)
        out_c.append(c)
        out_s.append(s)
    n = qb.shape[1]
    c = np.concatenate(out_c) if out_c else np.zeros((0, n))
    s = np.concatenate(out_s) if out_s else np.zeros((0, n))
    return rows, c, s


def grouped_masked_ref(qa, sa, qb, sb, masked_m):
    """Masked MoE layout: expert g owns rows [0, masked_m[g]) of its padded buffer.

    qa u8 [G][M_max][K], sa [G][K/128][M_max], qb u8 [G][N][K], sb [G][N/128][K/128].
    Returns a list of (C_ref, S) per expert, each [masked_m[g]][N].
    """
    res = []
    for g, m in enumerate(np.asarray(masked_m, dtype=np.int64)):
        rows = np.arange(int(m))
        res.append(gemm_blockscaled_ref(qa[g], sa[g], qb[g], sb[g], "128x128", rows=rows))
    return res
