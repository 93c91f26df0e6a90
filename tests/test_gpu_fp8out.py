"""GPU tests of the GEMM with the fused 1x128 output quantization.

Where the GEMM's FP32 result is exact (one nonzero product per output), the
fused codes and scales must equal the oracle's quantization of the exact C
bit for bit.  Elsewhere C is only known within the GEMM bound, so several
quantizations are correct: each scale must be one an output inside the bound
could give, and each code must decode to within the bound plus one E4M3 step
of the exact value.  All inputs come from the oracle or the seeded generators."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amd as fp8
from oracle import e4m3, gemm, quant
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _identity_case(rng, M, N, unit_scales):
    K = N
    qa = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x00
    # unit or power-of-two scales: the accumulator's unit is then 1 in every
    # K-block, so no rescale rounds (other scales keep C only within the bound)
    sa = np.ones((K // 128, M), np.float32) if unit_scales else \
        (2.0 ** rng.integers(-20, 21, size=(K // 128, M))).astype(np.float32)
    qb = np.where(np.eye(N, K, dtype=bool), np.uint8(0x38), np.uint8(0)).astype(np.uint8)
    sb = np.ones((N // 128, K // 128), np.float32)
    # C = RN32(dec(qa) * sa): one nonzero product per output, one rounding; the
    # other K - 1 products are +0, so an output whose code is -0 sums to +0
    c_exact = quant.dequant32(qa, np.repeat(sa.T, 128, axis=1)) + np.float32(0.0)
    return qa, sa, qb, sb, c_exact


@pytest.mark.parametrize("unit_scales", [True, False])
@pytest.mark.parametrize("M", [300, 64])
def test_exact_outputs_quantize_bit_for_bit(M, unit_scales):
    rng = np.random.default_rng(M + int(unit_scales))
    qa, sa, qb, sb, c_exact = _identity_case(rng, M, 512, unit_scales)
    q, s = fp8.fp8_gemm_blockscaled_fp8out(dev(qa), dev(sa), dev(qb), dev(sb))
    oq, os_ = quant.quant_act_1x128(c_exact)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))
    gq = host(q)
    bad = np.argwhere(gq != oq)
    assert bad.size == 0, [(tuple(i), hex(gq[tuple(i)]), hex(oq[tuple(i)]), float(c_exact[tuple(i)]))
                           for i in bad[:6]]
    # and the FP32 output of the same GEMM is that exact C
    c = fp8.fp8_gemm_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_128x128, torch.float32)
    assert np.array_equal(host(c).view(np.uint32), c_exact.view(np.uint32))


def _check_valid(q, s, c_ref, s_abs, what):
    """q u8 [R][N], s [N/128][R] against the exact C (rows of c_ref)."""
    R, N = c_ref.shape
    lim = gemm.bound(c_ref, s_abs, "fp32")
    g_ref = np.abs(c_ref).reshape(R, N // 128, 128)
    g_lim = lim.reshape(R, N // 128, 128)
    amax = g_ref.max(axis=2)
    slack = (g_ref + g_lim).max(axis=2) - amax          # how far the GPU's amax can exceed the exact one
    lo = (np.maximum(amax - g_lim.max(axis=2), 0) / 448.0).astype(np.float32)
    hi = ((amax + slack) / 448.0).astype(np.float32)
    st = s.T                                              # [R][N/128]
    bad = np.argwhere((st < np.nextafter(lo, np.float32(0))) | (st > np.nextafter(hi, np.float32(np.inf))))
    assert bad.size == 0, f"{what}: scales outside [{lo[tuple(bad[0])]}, {hi[tuple(bad[0])]}]: {st[tuple(bad[0])]}"
    s_full = np.repeat(st, 128, axis=1).astype(np.float64)
    val = e4m3.decode(q) * s_full
    y_hi = (np.abs(c_ref) + lim) / np.where(s_full > 0, s_full, 1.0)
    step = e4m3.ulp_at(y_hi) * s_full
    err = np.abs(val - c_ref)
    badc = np.argwhere(err > lim + step)
    assert badc.size == 0, f"{what}: {len(badc)} codes off, first {badc[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(200, 512, 1040), (257, 256, 128)])
def test_random_outputs_are_valid_quantizations(M, N, K):
    rng = np.random.default_rng(M + N + K)
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    q, s = fp8.fp8_gemm_blockscaled_fp8out(dev(qa), dev(sa), dev(qb), dev(sb))
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128")
    _check_valid(host(q), host(s), c_ref, s_abs, f"fp8out {M}x{N}x{K}")


def test_full_size_dense_fprop():
    x, w = workloads.dense_fprop()
    qa, sa = quant.quant_act_1x128(x)
    qb, sb = quant.quant_weight_128x128(w)
    q, s = fp8.fp8_gemm_blockscaled_fp8out(dev(qa), dev(sa), dev(qb), dev(sb))
    rows = np.concatenate([np.random.default_rng(8).choice(4096, 64, replace=False), [0, 4095]])
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128", rows=rows)
    _check_valid(host(q)[rows], host(s)[:, rows], c_ref, s_abs, "fp8out full size")
