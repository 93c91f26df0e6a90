"""Pins for the oracle's GEMM reference and acceptance bound (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import accum, e4m3, gemm, quant
from tests.goldens import gemm_hand_case
import workloads


def _code_fraction(c):
    """Exact rational value of an E4M3 code, from the bit fields."""
    s, e, m = c >> 7, (c >> 3) & 0xF, c & 7
    v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def _brute_force(qa, sa, qb, sb, bscale_kind, cols):
    """C[m][n] for n in cols: sum_k dec(qa)*sA * dec(qb)*sB with Python rationals."""
    M, K = qa.shape
    C = {}
    for m in range(M):
        for n in cols:
            acc = Fraction(0)
            for k in range(K):
                kb = k // 128
                av = _code_fraction(int(qa[m, k])) * Fraction(float(sa[kb, m]))
                sbv = sb[n // 128, kb] if bscale_kind == "128x128" else sb[kb, n]
                acc += av * _code_fraction(int(qb[n, k])) * Fraction(float(sbv))
            C[m, n] = acc
    return C


@pytest.mark.parametrize("K", [256, 176])
@pytest.mark.parametrize("bscale_kind", ["128x128", "1x128"])
def test_reference_against_exact_rationals(bscale_kind, K):
    """Tiny shapes: the float64 reference agrees with exact rational arithmetic
    to within K * 2^-53 * S (K = 176: a partial last K-block of 48)."""
    rng = np.random.default_rng(20 + K)
    M, N = 3, (128 if bscale_kind == "128x128" else 4)
    a = workloads.activations(rng, M, K, 0.01, 50.0)
    if bscale_kind == "128x128":
        qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    else:
        qb, sb = quant.quant_act_1x128(workloads.activations(rng, N, K))
    qa, sa = quant.quant_act_1x128(a)
    cols = [0, 1, N - 1]
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, bscale_kind)
    exact = _brute_force(qa, sa, qb, sb, bscale_kind, cols)
    for (m, n), v in exact.items():
        err = abs(Fraction(float(c_ref[m, n])) - v)
        assert err <= Fraction(K) * Fraction(2) ** -53 * Fraction(float(s_abs[m, n]))
        assert c_ref[m, n] != 0


def test_hand_worked_gemm():
    a, b, exp = gemm_hand_case()
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    assert sa[0, 0] == 1.0 and sb[0, 0] == 1.0
    assert qa[0, 0] == 0x7E and np.all(qa[0, 1:] == 0x38)
    assert qb[0, 0] == 0x7E and np.all(qb[1:, :] == 0x30)
    c, _ = gemm.gemm_blockscaled_ref(qa, sa, qb, sb)
    assert c[0, 0] == exp[("fp32", "n0")] and np.all(c[0, 1:] == exp[("fp32", "n_other")])
    import torch
    cb = torch.from_numpy(c.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert cb[0, 0] == exp[("bf16", "n0")] and np.all(cb[0, 1:] == exp[("bf16", "n_other")])


def test_bound_separates_fp32_promotion_from_limited_accumulation():
    """The FP32 block-and-promote emulation sits well inside u*S; a 14-bit
    accumulator without promotion does not."""
    rng = np.random.default_rng(21)
    M, N, K = 8, 128, 2048
    a = workloads.activations(rng, M, K, 0.001, 100.0)
    b = workloads.weights(rng, N, K)
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb)
    c32 = accum.accum_fp32_promoted(qa, sa, qb, sb)
    lim = gemm.bound(c_ref, s_abs, "fp32")
    ratio = np.max(np.abs(c32 - c_ref) / lim)
    assert ratio < 2.0 ** -3
    c14 = accum.accum_limited(quant.dequant_act(qa, sa), quant.dequant_weight(qb, sb), 14, "rz")
    assert np.max(np.abs(c14 - c_ref) / lim) > 1.0
    # a BF16 rounding of the FP32 result passes the BF16 form of the bound
    import torch
    cb = torch.from_numpy(c32).to(torch.bfloat16).double().numpy()
    assert np.all(np.abs(cb - c_ref) <= gemm.bound(c_ref, s_abs, "bf16"))


def test_grouped_layouts_reduce_to_dense():
    rng = np.random.default_rng(22)
    G, N, K = 3, 128, 256
    counts = np.array([5, 0, 130])
    off = workloads.pad_offsets(counts)
    assert off.tolist() == [0, 128, 128, 384]
    a = workloads.activations(rng, int(off[-1]), K)
    qa, sa = quant.quant_act_1x128(a)
    qbs, sbs = zip(*[quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    rows, c, s = gemm.grouped_contiguous_ref(qa, sa, qb, sb, off)
    assert rows.tolist() == list(range(384))
    for g in range(G):
        lo, hi = off[g], off[g + 1]
        if hi > lo:
            cd, _ = gemm.gemm_blockscaled_ref(qa[lo:hi], sa[:, lo:hi], qb[g], sb[g])
            assert np.array_equal(c[lo:hi], cd)
    mm = np.array([1, 64, 17])
    qam = np.stack([qa[:128], qa[128:256], qa[256:384]])
    sam = np.stack([sa[:, :128], sa[:, 128:256], sa[:, 256:384]])
    res = gemm.grouped_masked_ref(qam, sam, qb, sb, mm)
    for g in range(G):
        assert res[g][0].shape == (mm[g], N)
        cd, _ = gemm.gemm_blockscaled_ref(qam[g][:mm[g]], sam[g][:, :mm[g]], qb[g], sb[g])
        assert np.array_equal(res[g][0], cd)
