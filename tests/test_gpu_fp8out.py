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
from oracle import e4m3, gemm, layout, quant
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


# ---------------------------------------------------------------------------
# The contiguous MoE layout with the fused output quantization (the gate+up
# output feeding the down projection as its 1x128 A operand).

def test_contiguous_exact_outputs_quantize_bit_for_bit():
    """Identity experts (one nonzero product per output, power-of-two A
    scales): codes and scales equal the oracle's quantization of the exact C;
    rows in no expert's range keep the zeros they had."""
    rng = np.random.default_rng(61)
    N = K = 512
    off = np.array([0, 256, 384, 384], np.int32)     # experts of 256, 128 and 0 rows; rows 384-511 in none
    M = 512
    qa = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x00
    sa = (2.0 ** rng.integers(-20, 21, size=(K // 128, M))).astype(np.float32)
    eye = np.where(np.eye(N, K, dtype=bool), np.uint8(0x38), np.uint8(0)).astype(np.uint8)
    qb = np.stack([eye] * 3)
    sb = np.ones((3, N // 128, K // 128), np.float32)
    c_exact = quant.dequant32(qa, np.repeat(sa.T, 128, axis=1)) + np.float32(0.0)
    q, s = fp8.fp8_grouped_gemm_contiguous_fp8out(dev(qa), dev(sa), dev(qb), dev(sb), dev(off))
    oq, os_ = quant.quant_act_1x128(c_exact[:384])
    gq, gs = host(q), host(s)
    assert np.array_equal(gs[:, :384].view(np.uint32), os_.view(np.uint32))
    bad = np.argwhere(gq[:384] != oq)
    assert bad.size == 0, [(tuple(i), hex(gq[tuple(i)]), hex(oq[tuple(i)])) for i in bad[:6]]
    assert not gq[384:].any() and not gs[:, 384:].any(), "rows outside every expert were written"


@pytest.mark.parametrize("K", [384, 1040])
def test_contiguous_fp8out_is_the_quantized_fp32_output(K):
    """Ragged experts (5, 0, 300, 128 and 1 routed rows, each padded to 128),
    K with and without a partial last K-block: the fused codes and scales are
    the 1x128 quantizer applied to the FP32 output of the same GEMM, bit for
    bit, and a valid quantization of the oracle's C within the GEMM bound."""
    rng = np.random.default_rng(62 + K)
    counts = np.array([5, 0, 300, 128, 1])
    off = workloads.pad_offsets(counts)
    G, N = 5, 512
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, int(off[-1]), K, 0.01, 100.0))
    qs, ss = zip(*[quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)])
    qb, sb = np.stack(qs), np.stack(ss)
    args = [dev(qa), dev(sa), dev(qb), dev(sb), dev(off.astype(np.int32))]
    q, s = fp8.fp8_grouped_gemm_contiguous_fp8out(*args)
    c = fp8.fp8_grouped_gemm_contiguous(*args, torch.float32)
    rq, rs = fp8.fp8_quant_act_1x128(c)
    torch.cuda.synchronize()
    assert torch.equal(q, rq)
    assert torch.equal(s.view(torch.int32), rs.view(torch.int32))
    rows, cr, s_abs = gemm.grouped_contiguous_ref(qa, sa, qb, sb, off)
    _check_valid(host(q)[rows], host(s)[:, rows], cr, s_abs, f"contiguous fp8out K={K}")


@pytest.mark.timeout(900)
def test_contiguous_fp8out_full_size():
    """The MoE gate+up layer (32 experts, 65536 Zipf-routed rows padded per
    expert, N=4096, K=7168): equal to the quantized FP32 output everywhere,
    and sampled rows (each expert's first and last, plus random ones) valid
    against the oracle."""
    counts, off = workloads.moe_contig_layout()
    G, N, K = 32, 4096, 7168
    a = workloads.moe_contig_rows(counts, off, K)
    qa, sa = quant.quant_act_1x128(a)
    del a
    qs, ss = zip(*[quant.quant_weight_128x128(workloads.expert_weight("moe_gate_up", g, N, K)) for g in range(G)])
    qb, sb = np.stack(qs), np.stack(ss)
    del qs, ss
    args = [dev(qa), dev(sa), dev(qb), dev(sb), dev(off.astype(np.int32))]
    q, s = fp8.fp8_grouped_gemm_contiguous_fp8out(*args)
    c = fp8.fp8_grouped_gemm_contiguous(*args, torch.float32)
    rq, rs = fp8.fp8_quant_act_1x128(c)
    torch.cuda.synchronize()
    assert torch.equal(q, rq)
    assert torch.equal(s.view(torch.int32), rs.view(torch.int32))
    del c, rq, rs, args
    rng = np.random.default_rng(63)
    rows = [[off[g], off[g + 1] - 1] for g in range(G) if off[g + 1] > off[g]]
    rows = np.unique(np.concatenate([np.concatenate(rows), rng.integers(0, int(off[-1]), 64)]))
    sel, cr, s_abs = gemm.grouped_contiguous_ref(qa, sa, qb, sb, off, rows=rows)
    _check_valid(host(q)[sel], host(s)[:, sel], cr, s_abs, "contiguous fp8out full size")


# ---------------------------------------------------------------------------
# The masked decode layout on decode-tiled weights with the fused output
# quantization (fp8_grouped_gemm_masked_tiled_fp8out): codes u8 [G][M_max][N],
# scales f32 [G][N/128][M_max], the masked A operand's own layout.

def _masked_tiled_fp8out(qa, sa, qb, sb, mm):
    args = [dev(qa), dev(sa), dev(layout.tile_weights_decode(qb)), dev(sb), dev(np.asarray(mm, np.int32))]
    q, s = fp8.fp8_grouped_gemm_masked_tiled_fp8out(*args)
    return args, q, s


@pytest.mark.parametrize("N", [512, 768])
def test_masked_tiled_exact_outputs_quantize_bit_for_bit(N):
    """Identity experts (one nonzero product per output, power-of-two A
    scales), 512-column items (N = 512) and 256-column items (N = 768): the
    valid rows' codes and scales equal the oracle's quantization of the exact
    C; rows past masked_m keep the zeros they had."""
    rng = np.random.default_rng(64 + N)
    G, M_max, K = 4, 128, N
    mm = np.array([128, 0, 1, 77])
    qa = rng.integers(0, 256, size=(G, M_max, K), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x00
    sa = (2.0 ** rng.integers(-20, 21, size=(G, K // 128, M_max))).astype(np.float32)
    eye = np.where(np.eye(N, K, dtype=bool), np.uint8(0x38), np.uint8(0)).astype(np.uint8)
    qb = np.stack([eye] * G)
    sb = np.ones((G, N // 128, K // 128), np.float32)
    _, q, s = _masked_tiled_fp8out(qa, sa, qb, sb, mm)
    gq, gs = host(q), host(s)
    for g in range(G):
        m = int(mm[g])
        c_exact = quant.dequant32(qa[g], np.repeat(sa[g].T, 128, axis=1)) + np.float32(0.0)
        if m:
            oq, os_ = quant.quant_act_1x128(c_exact[:m])
            assert np.array_equal(gs[g][:, :m].view(np.uint32), os_.view(np.uint32)), g
            bad = np.argwhere(gq[g, :m] != oq)
            assert bad.size == 0, (g, [(tuple(i), hex(gq[g][tuple(i)]), hex(oq[tuple(i)])) for i in bad[:6]])
        assert not gq[g, m:].any() and not gs[g][:, m:].any(), f"g={g}: rows past masked_m were written"


@pytest.mark.parametrize("G,M_max,N,K", [(6, 128, 1024, 448), (5, 96, 768, 320), (3, 64, 256, 64)])
def test_masked_tiled_fp8out_is_the_quantized_fp32_output(G, M_max, N, K):
    """Ragged valid counts (M_max, 0, 1, 33, ...): the fused codes and scales
    are the 1x128 quantizer applied to the FP32 output of the same GEMM, bit
    for bit, on every valid row, and a valid quantization of the oracle's C."""
    rng = np.random.default_rng(G * 10 + M_max + N + K)
    mm = rng.integers(0, M_max + 1, G)
    mm[:min(G, 4)] = [M_max, 0, 1, 33][:min(G, 4)]
    qa, sa = zip(*[quant.quant_act_1x128(workloads.activations(rng, M_max, K, 0.01, 50.0)) for _ in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    qs, ss = zip(*[quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)])
    qb, sb = np.stack(qs), np.stack(ss)
    args, q, s = _masked_tiled_fp8out(qa, sa, qb, sb, mm)
    c = fp8.fp8_grouped_gemm_masked_tiled(*args, torch.float32)
    res = gemm.grouped_masked_ref(qa, sa, qb, sb, mm)
    for g in range(G):
        m = int(mm[g])
        if m == 0:
            assert not bool(q[g].any()) and not bool(s[g].any()), g
            continue
        rq, rs = fp8.fp8_quant_act_1x128(c[g, :m].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(q[g, :m], rq), g
        assert torch.equal(s[g][:, :m].contiguous().view(torch.int32), rs.view(torch.int32)), g
        assert not bool(q[g, m:].any()) and not bool(s[g][:, m:].any()), g
        _check_valid(host(q[g, :m]), host(s[g][:, :m]), res[g][0], res[g][1], f"masked fp8out g={g}")


@pytest.mark.timeout(900)
def test_masked_tiled_fp8out_full_size_down():
    """The masked decode down projection (32 experts, 128-row buffers, rows
    U{1..64}, N = 7168, K = 2048): equal to the quantized FP32 output on every
    valid row, and sampled rows of every expert valid against the oracle."""
    G, M_max, N, K = 32, 128, 7168, 2048
    mm, a = workloads.moe_masked_inputs(N, K, G, M_max)
    qa, sa = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    del a
    qs, ss = zip(*[quant.quant_weight_128x128(workloads.expert_weight("moe_down", g, N, K)) for g in range(G)])
    qb, sb = np.stack(qs), np.stack(ss)
    del qs, ss
    args, q, s = _masked_tiled_fp8out(qa, sa, qb, sb, mm)
    c = fp8.fp8_grouped_gemm_masked_tiled(*args, torch.float32)
    rng = np.random.default_rng(65)
    for g in range(G):
        m = int(mm[g])
        rq, rs = fp8.fp8_quant_act_1x128(c[g, :m].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(q[g, :m], rq), g
        assert torch.equal(s[g][:, :m].contiguous().view(torch.int32), rs.view(torch.int32)), g
        assert not bool(q[g, m:].any()) and not bool(s[g][:, m:].any()), g
        rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 3)]))
        cr, s_abs = gemm.gemm_blockscaled_ref(qa[g], sa[g], qb[g], sb[g], rows=rows)
        _check_valid(host(q[g])[rows], host(s[g])[:, rows], cr, s_abs, f"masked fp8out full g={g}")
