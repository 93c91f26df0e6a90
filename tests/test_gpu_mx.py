"""GPU parity of the MX variant against the oracle: quantizer codes and scale
bytes bit for bit; GEMM within the FP8-MFMA bound (u = 2^-9, the
instruction's limited in-group accumulation) plus the BF16 rounding.  Inputs
of the GEMM tests are MX-quantized by the oracle on the host."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amd as fp8
from oracle import gemm, mx
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U_MX = 2.0 ** -9
BF16_UNIT = 2.0 ** -8


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _inputs(rng, R, K):
    x = (rng.standard_normal((R, K)) * np.exp(rng.uniform(-6, 6, size=(R, 1)))).astype(np.float32)
    if R > 2 and K >= 96:
        x[0, :32] = 0.0
        x[0, 3] = -0.0
        x[1, 32:64] = np.float32(1.9)                           # saturation
        x[2, 64:96] = np.float32(2.0 ** -130) * np.arange(32)   # subnormal block: scale clamps
    return x


@pytest.mark.parametrize("R,K", [(1, 32), (5, 96), (64, 256), (257, 1024), (3, 4128)])
def test_quant_mx_bit_exact(R, K):
    x = _inputs(np.random.default_rng(R * 7 + K), R, K)
    q, e = fp8.fp8_quant_mx_1x32(dev(x))
    oq, oe = mx.quant_mx_1x32(x)
    assert np.array_equal(host(e), oe)
    bad = np.argwhere(host(q) != oq)
    assert bad.size == 0, bad[:5].tolist()


def _check(c, a_dq, b_dq, out, what):
    c_ref, s_abs = gemm.gemm_ref(a_dq, b_dq)
    lim = U_MX * s_abs if out == "fp32" else U_MX * s_abs * (1 + BF16_UNIT) + BF16_UNIT * np.abs(c_ref)
    err = np.abs(c - c_ref)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, f"{what}: {len(bad)} outside, max err/bound {np.max(err / np.maximum(lim, 1e-300)):.3g}"
    return float(np.max(err / np.maximum(s_abs, 1e-300)))


@pytest.mark.parametrize("M,N,K", [(4, 256, 64), (100, 512, 1024), (256, 256, 128), (260, 768, 2048)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_gemm_mx_bound(M, N, K, out):
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    a = workloads.activations(rng, M, K, 0.01, 50.0)
    b = workloads.weights(rng, N, K)
    qa, ea = mx.quant_mx_1x32(a)
    qb, eb = mx.quant_mx_1x32(b)
    c = fp8.fp8_gemm_mx(dev(qa), dev(ea), dev(qb), dev(eb), torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    _check(c.float().cpu().numpy().astype(np.float64), mx.dequant_mx(qa, ea), mx.dequant_mx(qb, eb), out,
           f"mx {M}x{N}x{K} {out}")


def test_gemm_mx_scales_are_applied_per_block():
    """Codes all 1.0 (0x38) and scale bytes that differ per 32-K block and per
    row: every product is a power of two within 2^4 of the others, so even the
    instruction's limited-width sums are exact, and C must equal the exact
    value bit for bit (FP32 out).  A scale applied to the wrong block or row
    changes the sum."""
    rng = np.random.default_rng(12)
    M, N, K = 64, 256, 256
    qa = np.full((M, K), 0x38, np.uint8)
    qb = np.full((N, K), 0x38, np.uint8)
    ea = rng.integers(126, 129, size=(K // 32, M)).astype(np.uint8)
    eb = rng.integers(126, 129, size=(K // 32, N)).astype(np.uint8)
    c = fp8.fp8_gemm_mx(dev(qa), dev(ea), dev(qb), dev(eb), torch.float32)
    ref = mx.dequant_mx(qa, ea) @ mx.dequant_mx(qb, eb).T
    assert np.array_equal(host(c).astype(np.float64), ref)


def test_gemm_mx_full_size_dense_fprop():
    """The 4096x7168x2048 workload, MX-quantized; sampled rows checked."""
    x, w = workloads.dense_fprop()
    qa, ea = mx.quant_mx_1x32(x)
    qb, eb = mx.quant_mx_1x32(w)
    c = fp8.fp8_gemm_mx(dev(qa), dev(ea), dev(qb), dev(eb), torch.bfloat16)
    rows = np.random.default_rng(5).choice(4096, size=96, replace=False)
    rows = np.concatenate([rows, [0, 255, 256, 4095]])
    torch.cuda.synchronize()
    cg = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    a_dq = mx.dequant_mx(qa, ea)[rows]
    _check(cg, a_dq, mx.dequant_mx(qb, eb), "bf16", "mx full size")
    # the GPU quantizer gives the same operands
    gq, ge = fp8.fp8_quant_mx_1x32(dev(x))
    assert np.array_equal(host(gq), qa) and np.array_equal(host(ge), ea)
