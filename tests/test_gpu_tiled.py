"""GPU parity of the decode-tiled weight layout and of the masked GEMM that
reads it.

fp8_tile_weights_decode is a byte permutation: it must equal the oracle's
(oracle/layout.py) byte for byte.  fp8_grouped_gemm_masked_tiled runs a
different kernel (persistent, weight fragments streamed into registers) with
the same arithmetic as fp8_grouped_gemm_masked -- the same fragments, map of
k to MFMA steps and unit fold -- so it must equal that GEMM on the plain
layout bit for bit, and stay inside the oracle GEMM's bound; rows past
masked_m are not written."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amd as fp8
from oracle import gemm, layout, quant
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
OUT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _same_bits(c1, c0):
    a, b = c1.cpu(), c0.cpu()
    return torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("G,N,K", [(1, 256, 64), (3, 512, 320), (2, 768, 2048)])
def test_tile_weights_matches_oracle(G, N, K):
    rng = np.random.default_rng(G * 7 + N + K)
    q = rng.integers(0, 256, (G, N, K), dtype=np.uint8)
    t = fp8.fp8_tile_weights_decode(dev(q))
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), layout.tile_weights_decode(q))


def test_tile_weights_full_size_sampled():
    """The gate+up experts (32 x 4096 x 7168): three experts against the oracle."""
    G, N, K = 32, 4096, 7168
    g = torch.Generator(device=DEV).manual_seed(11)
    q = torch.randint(0, 256, (G, N, K), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    t = fp8.fp8_tile_weights_decode(q)
    torch.cuda.synchronize()
    for e in (0, 17, 31):
        assert np.array_equal(t[e:e + 1].cpu().numpy(), layout.tile_weights_decode(q[e:e + 1].cpu().numpy())), e


# (G, M_max, N, K, out): whole K-blocks; K = 128 q + 64 (a last half K-block);
# one half-block; 96-row buffers; fp32 out; a last half K-block with N a
# multiple of 512 (eight-wave items) and with a 256-wide item (N = 256 mod 512)
@pytest.mark.parametrize("G,M_max,N,K,out", [(8, 128, 512, 384, "bf16"), (5, 64, 768, 320, "fp32"),
                                             (4, 100, 256, 64, "bf16"), (8, 96, 1024, 1152, "fp32"),
                                             (6, 128, 1024, 448, "bf16"), (4, 128, 512, 64, "fp32"),
                                             # items of 448 columns (seven-wave workgroups)
                                             (8, 128, 1792, 448, "bf16"), (8, 128, 1792, 384, "fp32"),
                                             (4, 128, 3584, 192, "fp32")])
def test_masked_tiled_matches_plain_and_oracle(G, M_max, N, K, out):
    rng = np.random.default_rng(G * 100 + M_max + N + K)
    mm = rng.integers(0, M_max + 1, G).astype(np.int32)
    mm[:4] = [M_max, 0, 1, 33]
    a = np.stack([workloads.activations(rng, M_max, K, 0.01, 50.0) for _ in range(G)])
    qa, sa = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    qs, ss = zip(*[quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)])
    qb, sb = np.stack(qs), np.stack(ss)
    sa[0, 0, 5] = 0.0        # a zero A scale: that row's first K-block reads as zero
    sb[3, -1, -1] = 0.0      # a zero B scale in the last n-block and K-block
    qt = dev(layout.tile_weights_decode(qb))
    args = dict(a=dev(qa), sa=dev(sa), sb=dev(sb), masked_m=dev(mm))
    c_t = torch.full((G, M_max, N), -9.0, dtype=OUT[out], device=DEV)
    fp8.fp8_grouped_gemm_masked_tiled(args["a"], args["sa"], qt, args["sb"], args["masked_m"], OUT[out], out=c_t)
    c_p = torch.full((G, M_max, N), -9.0, dtype=OUT[out], device=DEV)
    fp8.fp8_grouped_gemm_masked(args["a"], args["sa"], dev(qb), args["sb"], args["masked_m"], OUT[out], out=c_p)
    torch.cuda.synchronize()
    assert _same_bits(c_t, c_p), "the tiled layout changed the result"
    res = gemm.grouped_masked_ref(qa, sa, qb, sb, mm)
    ch = c_t.double().cpu().numpy()
    for g in range(G):
        m = int(mm[g])
        err = np.abs(ch[g, :m] - res[g][0])
        assert np.all(err <= gemm.bound(res[g][0], res[g][1], out)), g
        assert np.all(ch[g, m:] == -9.0), f"g={g}: rows past masked_m were written"


@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)])
def test_masked_tiled_full_size_matches_plain(N, K):
    """The masked decode shapes (32 experts, 128-row buffers, rows U{1..64}),
    tiled by the GPU: the same bits as the plain layout.  Operands come from
    the GPU quantizers (this compares two GPU paths; the oracle parity of these
    shapes is in test_gpu_gemm)."""
    G, M_max = 32, 128
    g = torch.Generator(device=DEV).manual_seed(N * 3 + K)
    x = torch.randn((G * M_max, K), generator=g, device=DEV)
    qa, sa = fp8.fp8_quant_act_1x128(x)
    qa = qa.view(G, M_max, K)
    sa = sa.view(K // 128, G, M_max).permute(1, 0, 2).contiguous()
    qb = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    sb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=DEV)
    for e in range(G):
        qb[e], sb[e] = fp8.fp8_quant_weight_128x128(torch.randn((N, K), generator=g, device=DEV) * 0.02)
    mm = torch.randint(1, 65, (G,), generator=g, device=DEV, dtype=torch.int32)
    qt = fp8.fp8_tile_weights_decode(qb)
    c_t = torch.full((G, M_max, N), 5.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_masked_tiled(qa, sa, qt, sb, mm, out=c_t)
    c_p = torch.full((G, M_max, N), 5.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_masked(qa, sa, qb, sb, mm, out=c_p)
    torch.cuda.synchronize()
    assert _same_bits(c_t, c_p)
