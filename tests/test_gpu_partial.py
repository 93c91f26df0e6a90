"""GPU parity with partial groups: the grouped axis (K, or the token axis of
the token-wise layout) or N a multiple of 16 but not of 128.  Quantizers bit for
bit against the oracle (which quantizes the zero-padded group); GEMMs within
the usual bounds, on every kernel family (wide, decode, fold, the FP8-MFMA
engine, 1x128-scaled B, both grouped layouts)."""
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


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host64(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def bf16_pair(x):
    bits = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return (torch.from_numpy((bits >> np.uint32(16)).astype(np.uint16)).to(DEV).view(torch.bfloat16),
            (bits & np.uint32(0xFFFF0000)).view(np.float32))


def same(gq, gs, oq, os_, what):
    gq, gs = host(gq), host(gs)
    bad = np.argwhere(gq != oq)
    assert bad.size == 0, f"{what}: {len(bad)} code mismatches, first {bad[:3].tolist()}"
    assert np.array_equal(gs.view(np.uint32), np.asarray(os_, np.float32).view(np.uint32)), f"{what}: scales"


def check(c, c_ref, s_abs, out, what, u=gemm.U):
    lim = u * s_abs if out == "fp32" else u * s_abs * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(c_ref)
    err = np.abs(c - c_ref)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, f"{what}: {len(bad)} outside, max err/bound {np.max(err / np.maximum(lim, 1e-300)):.3g}"


@pytest.mark.parametrize("M,K", [(5, 16), (7, 208), (300, 1040), (33, 7216)])
def test_rows_partial(M, K):
    x = workloads.activations(np.random.default_rng(M + K), M, K, 0.02, 80.0)
    same(*fp8.fp8_quant_act_1x128(dev(x)), *quant.quant_act_1x128(x), f"rows {M}x{K}")
    xb, xw = bf16_pair(x)
    same(*fp8.fp8_quant_act_1x128_bf16(xb), *quant.quant_act_1x128(xw), f"bf16 rows {M}x{K}")


@pytest.mark.parametrize("M,K", [(16, 64), (144, 100), (400, 333), (272, 2048)])
def test_tokens_partial(M, K):
    x = workloads.activations(np.random.default_rng(3 * M + K), M, K, 0.02, 80.0)
    same(*fp8.fp8_quant_act_1x128(dev(x), transpose_out=True), *quant.quant_act_1x128_tokenwise(x),
         f"tokens {M}x{K}")
    xb, xw = bf16_pair(x)
    same(*fp8.fp8_quant_act_1x128_bf16(xb, transpose_out=True), *quant.quant_act_1x128_tokenwise(xw),
         f"bf16 tokens {M}x{K}")


@pytest.mark.parametrize("N,K", [(128, 16), (256, 208), (384, 1040)])
@pytest.mark.parametrize("transpose", [False, True])
def test_weight_partial(N, K, transpose):
    w = workloads.weights(np.random.default_rng(N + 5 * K), N, K)
    w[N - 1, K - 1] = 1.5                            # the partial block's max sits in its last column
    same(*fp8.fp8_quant_weight_128x128(dev(w), transpose_out=transpose),
         *quant.quant_weight_128x128(w, transpose_out=transpose), f"weight {N}x{K} T={transpose}")
    wb, ww = bf16_pair(w)
    same(*fp8.fp8_quant_weight_128x128_bf16(wb, transpose_out=transpose),
         *quant.quant_weight_128x128(ww, transpose_out=transpose), f"bf16 weight {N}x{K} T={transpose}")


@pytest.mark.parametrize("M,K", [(144, 208), (16, 16), (528, 1040)])
def test_requant_partial(M, K):
    x = workloads.activations(np.random.default_rng(M * K), M, K, 0.02, 80.0)
    q, s = quant.quant_act_1x128(x)
    same(*fp8.fp8_requant_act_tokenwise(dev(q), dev(s)), *quant.requant_act_tokenwise(q, s),
         f"requant {M}x{K}")


@pytest.mark.parametrize("M,N,K", [(100, 256, 208), (300, 512, 1040), (64, 384, 176), (257, 256, 16)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_dense_partial_k(M, N, K, out):
    """N % 256 == 0 runs the wide kernel, N = 384 the fold kernel."""
    rng = np.random.default_rng(M + N + K)
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    c = fp8.fp8_gemm_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_128x128, OUT[out])
    check(host64(c), *gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128"), out, f"dense {M}x{N}x{K} {out}")


@pytest.mark.parametrize("M,N,K", [(128, 256, 144), (256, 384, 1040)])
def test_wgrad_partial_tokens(M, N, K):
    """1x128-scaled B (the Wgrad layout; K = tokens, a multiple of 16)."""
    rng = np.random.default_rng(M + N + K + 1)
    dy = workloads.activations(rng, K, M, 0.0, 1.0, 1e-3)      # [tokens][out]
    x = workloads.activations(rng, K, N, 0.01, 50.0)           # [tokens][in]
    qa, sa = quant.quant_act_1x128_tokenwise(dy)               # [out][tokens]
    qb, sb = quant.quant_act_1x128_tokenwise(x)                # [in][tokens]
    c = fp8.fp8_gemm_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_1x128, torch.float32)
    check(host64(c), *gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "1x128"), "fp32", f"wgrad {M}x{N}x{K}")


def test_fp8mfma_engine_partial_k():
    rng = np.random.default_rng(77)
    M, N, K = 130, 256, 336
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    c = fp8.fp8_gemm_blockscaled_fp8mfma(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_128x128, torch.float32)
    check(host64(c), *gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128"), "fp32", "fp8mfma partial",
          u=2.0 ** -9)


@pytest.mark.parametrize("N", [256, 384])
def test_grouped_partial_k(N):
    rng = np.random.default_rng(N)
    G, K = 3, 208
    counts = np.array([128, 0, 256])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = workloads.activations(rng, int(off[-1]), K, 0.01, 50.0)
    qa, sa = quant.quant_act_1x128(a)
    qbs = [quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    c = fp8.fp8_grouped_gemm_contiguous(dev(qa), dev(sa), dev(qb), dev(sb), dev(off), torch.float32)
    rows, cr, sr = gemm.grouped_contiguous_ref(qa, sa, qb, sb, off)
    check(host64(c)[rows], cr, sr, "fp32", f"contig N={N}")
    # masked: 128-row buffers (decode tile) and 256-row buffers
    for M_max, mm in ((128, [5, 128, 77]), (256, [200, 1, 256])):
        am = workloads.activations(rng, G * M_max, K, 0.01, 50.0).reshape(G, M_max, K)
        qs = [quant.quant_act_1x128(am[g]) for g in range(G)]
        qam = np.stack([q for q, _ in qs])
        sam = np.stack([s for _, s in qs])
        mmv = np.array(mm, np.int32)
        out = torch.full((G, M_max, N), 7.0, dtype=torch.float32, device=DEV)
        fp8.fp8_grouped_gemm_masked(dev(qam), dev(sam), dev(qb), dev(sb), dev(mmv), torch.float32, out=out)
        o = host64(out)
        for g in range(G):
            cr, sr = gemm.gemm_blockscaled_ref(qam[g][:mm[g]], sam[g][:, :mm[g]], qb[g], sb[g], "128x128")
            check(o[g, :mm[g]], cr, sr, "fp32", f"masked M_max={M_max} N={N} g={g}")
            assert np.all(o[g, mm[g]:] == 7.0)


def test_full_size_mla_like_k():
    """A 4096 x 7168 x 576 GEMM (576 = 4.5 K-blocks), sampled rows."""
    rng = np.random.default_rng(576)
    M, N, K = 4096, 7168, 576
    a = workloads.activations(rng, M, K, 0.001, 100.0)
    w = workloads.weights(rng, N, K)
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(w)
    c = fp8.fp8_gemm_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_128x128, torch.bfloat16)
    rows = np.concatenate([np.random.default_rng(1).choice(M, 64, replace=False), [0, M - 1]])
    cg = host64(c[torch.from_numpy(rows).to(DEV)])
    check(cg, *gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128", rows=rows), "bf16", "K=576")
    gq, gs = fp8.fp8_quant_act_1x128(dev(a))
    same(gq, gs, qa, sa, "K=576 activations")


# ---------------------------------------------------------------------------
# N (output channels, rows of B) a multiple of 16 but not of 128: partial
# 128x128 blocks along N, and the fold kernels' last n-tile holds fewer
# columns (no column past N is written).

@pytest.mark.parametrize("N,K", [(16, 128), (144, 208), (400, 1040)])
@pytest.mark.parametrize("transpose", [False, True])
def test_weight_partial_n(N, K, transpose):
    w = workloads.weights(np.random.default_rng(7 * N + K), N, K)
    w[N - 1, 0] = -2.0
    same(*fp8.fp8_quant_weight_128x128(dev(w), transpose_out=transpose),
         *quant.quant_weight_128x128(w, transpose_out=transpose), f"weight N={N} K={K} T={transpose}")
    wb, ww = bf16_pair(w)
    same(*fp8.fp8_quant_weight_128x128_bf16(wb, transpose_out=transpose),
         *quant.quant_weight_128x128(ww, transpose_out=transpose), f"bf16 weight N={N} K={K} T={transpose}")


@pytest.mark.parametrize("M,N,K", [(100, 208, 256), (257, 400, 1040), (64, 16, 128)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_dense_partial_n(M, N, K, out):
    rng = np.random.default_rng(M + 3 * N + K)
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    c = torch.full((M + 1, N), 9.0, dtype=OUT[out], device=DEV)        # one guard row after C
    fp8.fp8_gemm_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_128x128, OUT[out], out=c[:M])
    cg = host64(c)
    check(cg[:M], *gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128"), out, f"dense N={N} {M}x{N}x{K}")
    assert np.all(cg[M] == 9.0)


def test_wgrad_partial_n_and_tokens():
    """1x128-scaled B with 144 output columns (in-features) and 208 tokens."""
    rng = np.random.default_rng(144)
    T, OUTF, INF = 208, 256, 144
    dy = workloads.activations(rng, T, OUTF, 0.0, 1.0, 1e-3)
    x = workloads.activations(rng, T, INF, 0.01, 50.0)
    qa, sa = quant.quant_act_1x128_tokenwise(dy)
    qb, sb = quant.quant_act_1x128_tokenwise(x)
    c = fp8.fp8_gemm_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_1x128, torch.float32)
    check(host64(c), *gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "1x128"), "fp32", "wgrad N=144")


def test_fp8mfma_engine_partial_n():
    rng = np.random.default_rng(88)
    M, N, K = 130, 176, 256
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    c = fp8.fp8_gemm_blockscaled_fp8mfma(dev(qa), dev(sa), dev(qb), dev(sb), fp8.BSCALE_128x128, torch.float32)
    check(host64(c), *gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128"), "fp32", "fp8mfma N=176",
          u=2.0 ** -9)


def test_grouped_partial_n():
    rng = np.random.default_rng(208)
    G, N, K = 3, 208, 256
    counts = np.array([256, 128, 0])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, int(off[-1]), K, 0.01, 50.0))
    qbs = [quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    c = fp8.fp8_grouped_gemm_contiguous(dev(qa), dev(sa), dev(qb), dev(sb), dev(off), torch.float32)
    rows, cr, sr = gemm.grouped_contiguous_ref(qa, sa, qb, sb, off)
    check(host64(c)[rows], cr, sr, "fp32", "contig N=208")
    for M_max, mm in ((128, [3, 128, 64]), (256, [256, 17, 0])):
        am = workloads.activations(rng, G * M_max, K, 0.01, 50.0).reshape(G, M_max, K)
        qs = [quant.quant_act_1x128(am[g]) for g in range(G)]
        qam = np.stack([q for q, _ in qs])
        sam = np.stack([s for _, s in qs])
        out = torch.full((G, M_max, N), 7.0, dtype=torch.float32, device=DEV)
        fp8.fp8_grouped_gemm_masked(dev(qam), dev(sam), dev(qb), dev(sb), dev(np.array(mm, np.int32)),
                                    torch.float32, out=out)
        o = host64(out)
        for g in range(G):
            if mm[g]:
                cr, sr = gemm.gemm_blockscaled_ref(qam[g][:mm[g]], sam[g][:, :mm[g]], qb[g], sb[g], "128x128")
                check(o[g, :mm[g]], cr, sr, "fp32", f"masked N=208 M_max={M_max} g={g}")
            assert np.all(o[g, mm[g]:] == 7.0)
