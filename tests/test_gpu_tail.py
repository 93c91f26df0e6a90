"""GPU parity of the dense GEMM's tail tiles: the 256 x 192 tiles that cover
the last columns of a dense grid whose 256 x 256 tiles would leave a partial
last round on the device.  They run the same per-K-block arithmetic in the
same order as the 256 x 256 tiles, so besides the oracle's bound the result
must equal, bit for bit, the same GEMM computed with 256 x 256 tiles only
(FP8FG_GEMM_TAIL=0).  FP8FG_GEMM_TAIL=force plans tail tiles on small shapes."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amd as fp8
from oracle import gemm, quant
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
OUT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _gemm(monkeypatch, tail, qa, sa, qb, sb, out):
    monkeypatch.setenv("FP8FG_GEMM_TAIL", tail)
    c = fp8.fp8_gemm_blockscaled(qa, sa, qb, sb, fp8.BSCALE_128x128, OUT[out])
    torch.cuda.synchronize()
    return c


def _same_bits(c1, c0):
    a, b = c1.cpu(), c0.cpu()
    return torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


# N = 256 a + 192 b with b > 0: 1024 = 256 + 4 x 192 (mixed), 768 = 4 x 192
# (tail tiles only), 1536 = 3 x 256 + 4 x 192; partial M and partial K
@pytest.mark.parametrize("M,N,K,out", [(300, 1024, 512, "bf16"), (64, 768, 176, "fp32"),
                                       (513, 1536, 1040, "bf16"), (256, 1024, 128, "fp32")])
def test_forced_tail_tiles(monkeypatch, M, N, K, out):
    rng = np.random.default_rng(M * 3 + N + K)
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    # zero scales: one row's first K-block, and the last n-block (tail columns)
    # in its first K-block: their codes must read as zero
    sa[0, min(5, M - 1)] = 0.0
    sb[-1, 0] = 0.0
    args = (dev(qa), dev(sa), dev(qb), dev(sb))
    c = _gemm(monkeypatch, "force", *args, out)
    c0 = _gemm(monkeypatch, "0", *args, out)
    assert _same_bits(c, c0), "tail tiles differ from the 256 x 256 tiles"
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128")
    err = np.abs(c.float().cpu().numpy().astype(np.float64) - c_ref)
    lim = gemm.bound(c_ref, s_abs, out)
    assert np.all(err <= lim), f"outside the bound: max err/bound {np.max(err / lim):.3g}"


@pytest.mark.parametrize("M,N,K", [(4096, 7168, 2048), (8192, 7168, 2048)])
def test_planned_tail_full_size_matches_full_tiles(monkeypatch, M, N, K):
    """The shapes whose 256 x 256 grid fills 256 CUs 1.75 and 3.5 times (the
    dense Fprop and the linear layer's Dgrad): the planned grid gives the same
    bits as the 256 x 256 grid.  Operands come from the GPU quantizers (this
    compares two GPU kernels; the oracle parity of these shapes is in
    test_gpu_gemm)."""
    g = torch.Generator(device=DEV).manual_seed(M + N)
    x = torch.randn((M, K), generator=g, device=DEV)
    w = torch.randn((N, K), generator=g, device=DEV) * 0.02
    qa, sa = fp8.fp8_quant_act_1x128(x)
    qb, sb = fp8.fp8_quant_weight_128x128(w)
    c0 = _gemm(monkeypatch, "0", qa, sa, qb, sb, "bf16")
    # the plan this device makes, and a forced split (tail tiles whatever the
    # CU count: N = 25 x 256 + 4 x 192)
    for mode in ("1", "force"):
        assert _same_bits(_gemm(monkeypatch, mode, qa, sa, qb, sb, "bf16"), c0), mode
