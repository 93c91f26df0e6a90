"""GPU parity of the block-scaled GEMMs against the CPU oracle.

Inputs are quantized by the oracle on the host and copied to the GPU, so no
GEMM input and no expected value comes from the HIP path.  Outputs must satisfy
the element-wise bound of oracle.gemm.bound (u = 2^-14); the exact special
cases must match bit for bit.  Full-size workloads are checked on sampled rows
(the oracle computes those rows exactly); everything else on all outputs.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amd as fp8
from oracle import e4m3, gemm, quant
from tests.goldens import gemm_hand_case
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
OUT = {"bf16": torch.bfloat16, "fp32": torch.float32}
BS = {"128x128": fp8.BSCALE_128x128, "1x128": fp8.BSCALE_1x128}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host64(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def check(c_gpu, c_ref, s_abs, out, what):
    err = np.abs(c_gpu - c_ref)
    lim = gemm.bound(c_ref, s_abs, out)
    bad = np.argwhere(err > lim)
    ratio = float(np.max(err / np.maximum(lim, 1e-300))) if err.size else 0.0
    assert bad.size == 0, f"{what}: {len(bad)} outputs outside the bound (max err/bound {ratio:.3g}), first {bad[:3].tolist()}"
    return ratio


def quant_b(b, kind):
    return quant.quant_weight_128x128(b) if kind == "128x128" else quant.quant_act_1x128(b)


def run_dense(qa, sa, qb, sb, kind, out):
    return fp8.fp8_gemm_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb), BS[kind], OUT[out])


def test_hand_worked_case():
    a, b, exp = gemm_hand_case()
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    for out in ("fp32", "bf16"):
        c = host64(run_dense(qa, sa, qb, sb, "128x128", out))
        assert c[0, 0] == exp[(out, "n0")] and np.all(c[0, 1:] == exp[(out, "n_other")]), out


def test_every_code_survives_the_gemm():
    """B = identity blocks with unit scales: C[m][n] = dec(A[m][n]) exactly, for
    every finite E4M3 code (checks the kernel's FP8 -> MFMA-operand path)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M, K = 2, 128 * 2
    qa = np.zeros((M, K), np.uint8)
    qa.reshape(-1)[:codes.size] = codes
    sa = np.ones((K // 128, M), np.float32)
    qb = np.zeros((K, K), np.uint8)
    np.fill_diagonal(qb, 0x38)                      # 1.0
    sb = np.ones((K // 128, K // 128), np.float32)
    c = host64(run_dense(qa, sa, qb, sb, "128x128", "fp32"))
    # values only: -0 * 1 plus the +0 products of the off-diagonal is +0
    assert np.array_equal(c, e4m3.decode(qa))


def test_exact_integer_case():
    """Tiles of small E4M3 integers with one 448 each: scales are exactly 1,
    every partial sum is an integer below 2^24, so FP32 output is exact and
    BF16 output is the round-to-nearest-even of the exact value."""
    rng = np.random.default_rng(40)
    M, N, K = 130, 256, 512
    ints = np.array([-16, -12, -8, -5, -3, -2, -1, 0, 1, 2, 3, 4, 6, 9, 13, 16], np.float32)
    a = rng.choice(ints, size=(M, K)).astype(np.float32)
    b = rng.choice(ints, size=(N, K)).astype(np.float32)
    a[:, ::128] = 448.0
    b[::128, ::128] = 448.0
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    assert np.all(sa == 1) and np.all(sb == 1)
    c_ref, _ = gemm.gemm_blockscaled_ref(qa, sa, qb, sb)
    assert np.all(np.abs(c_ref) < 2 ** 24)
    c32 = host64(run_dense(qa, sa, qb, sb, "128x128", "fp32"))
    assert np.array_equal(c32, c_ref)
    cbf = host64(run_dense(qa, sa, qb, sb, "128x128", "bf16"))
    ref_bf = torch.from_numpy(c_ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(cbf, ref_bf)


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 256, 256), (128, 256, 512), (130, 384, 384),
                                   (257, 128, 1024), (300, 512, 2048), (200, 512, 1040)])
@pytest.mark.parametrize("kind", ["128x128", "1x128"])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_dense_random(M, N, K, kind, out):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    a = workloads.activations(rng, M, K, 0.01, 50.0)
    b = workloads.weights(rng, N, K) if kind == "128x128" else workloads.activations(rng, N, K, 0.0, 1.0, 1e-3)
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant_b(b, kind)
    c = host64(run_dense(qa, sa, qb, sb, kind, out))
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, kind)
    check(c, c_ref, s_abs, out, f"dense {M}x{N}x{K} {kind} {out}")


def test_dense_small_workload():
    """128x256x512 with 0.5% outlier channels x50, BF16 out: every output checked."""
    a, b = workloads.dense_small()
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    c = host64(run_dense(qa, sa, qb, sb, "128x128", "bf16"))
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb)
    check(c, c_ref, s_abs, "bf16", "dense_small")
    c = host64(run_dense(qa, sa, qb, sb, "128x128", "fp32"))
    check(c, c_ref, s_abs, "fp32", "dense_small fp32")


def test_determinism_and_scale_linearity():
    rng = np.random.default_rng(41)
    a = workloads.activations(rng, 256, 1024, 0.01, 100.0)
    b = workloads.weights(rng, 384, 1024)
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    c1 = run_dense(qa, sa, qb, sb, "128x128", "fp32")
    c2 = run_dense(qa, sa, qb, sb, "128x128", "fp32")
    c4 = run_dense(qa, sa * np.float32(4.0), qb, sb, "128x128", "fp32")
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert torch.equal(c4, c1 * 4)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["128x128", "1x128"])
def test_scales_across_many_binades(out, kind):
    """Tile scales spread over 2^-64 .. 2^64 (A) and 2^-24 .. 2^24 (B), with
    one subnormal A scale: the promotion must hold for any scale pair, not
    just for quantizer-sized ones (the kernel splits scales into powers of two
    and mantissa parts, so this crosses all of its clamps)."""
    rng = np.random.default_rng(50)
    M, N, K = 300, 512, 1024
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    b = workloads.weights(rng, N, K) if kind == "128x128" else workloads.activations(rng, N, K, 0.01, 20.0, 1e-2)
    qb, sb = quant_b(b, kind)
    sa = (sa * np.exp2(rng.integers(-64, 65, sa.shape))).astype(np.float32)
    sb = (sb * np.exp2(rng.integers(-24, 25, sb.shape))).astype(np.float32)
    sa[3, 7] = np.float32(2.0 ** -140)
    if kind == "1x128":
        sb[2, 9] = np.float32(2.0 ** -135)     # a subnormal column scale
    c = host64(run_dense(qa, sa, qb, sb, kind, out))
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, kind)
    assert np.all(np.isfinite(c))
    check(c, c_ref, s_abs, out, f"scales across binades {kind} {out}")


@pytest.mark.parametrize("kind", ["128x128", "1x128"])
def test_zero_scales_with_nonzero_codes(kind):
    """A zero scale removes its block's products whatever the codes say: some
    A tiles and B blocks (or, 1x128 B, single columns of a K-block) get scale
    0 over nonzero codes, and row 5 has only zero scales, so its outputs must
    be exactly zero; with 1x128 B column 9 too."""
    rng = np.random.default_rng(51)
    M, N, K = 130, 512, 768
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    b = workloads.weights(rng, N, K) if kind == "128x128" else workloads.activations(rng, N, K, 0.01, 20.0, 1e-2)
    qb, sb = quant_b(b, kind)
    sa = sa.copy()
    sb = sb.copy()
    sa[rng.random(sa.shape) < 0.15] = 0.0
    sa[:, 5] = 0.0
    sb[rng.random(sb.shape) < 0.2] = 0.0
    if kind == "1x128":
        sb[:, 9] = 0.0
    for out in ("fp32", "bf16"):
        c = host64(run_dense(qa, sa, qb, sb, kind, out))
        c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, kind)
        check(c, c_ref, s_abs, out, f"zero scales {kind} {out}")
        assert np.all(c[5] == 0.0)
        if kind == "1x128":
            assert np.all(c[:, 9] == 0.0)


def sample_rows(M, rng, n=64):
    rows = np.concatenate([np.arange(min(M, 16)), np.arange(max(0, M - 16), M), rng.integers(0, M, n)])
    return np.unique(rows)


@pytest.mark.timeout(600)
def test_dense_fprop_full_size():
    """M=4096 N=7168 K=2048, BF16 out: sampled rows against the oracle."""
    x, w = workloads.dense_fprop()
    qa, sa = quant.quant_act_1x128(x)
    qb, sb = quant.quant_weight_128x128(w)
    c = run_dense(qa, sa, qb, sb, "128x128", "bf16")
    rows = sample_rows(4096, np.random.default_rng(42))
    c = host64(c[torch.from_numpy(rows).to(DEV)])
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, rows=rows)
    check(c, c_ref, s_abs, "bf16", "dense_fprop")


@pytest.mark.timeout(600)
def test_dense_fprop_full_size_fp32_literal_bound():
    """The headline shape (M=4096 N=7168 K=2048) with FP32 output, on the grid
    the dense call launches: sampled rows held to the literal element-wise
    bound |C - C*| <= 2^-14 S with no output-rounding term.  Prints the largest
    err / S seen, the engine's real margin."""
    x, w = workloads.dense_fprop()
    qa, sa = quant.quant_act_1x128(x)
    qb, sb = quant.quant_weight_128x128(w)
    c = run_dense(qa, sa, qb, sb, "128x128", "fp32")
    rows = sample_rows(4096, np.random.default_rng(142), 96)
    c = host64(c[torch.from_numpy(rows).to(DEV)])
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, rows=rows)
    check(c, c_ref, s_abs, "fp32", "dense_fprop fp32")
    rel = np.max(np.abs(c - c_ref) / np.maximum(s_abs, 1e-300))
    print(f"dense_fprop FP32: max |C - C*| / S = {rel:.3e} = 2^{np.log2(max(rel, 1e-300)):.2f} (bound 2^-14)")


@pytest.mark.parametrize("K", [92 * 128, 93 * 128])
def test_long_contraction_fp32_literal_bound(K):
    """The longest contraction the wide kernel takes (92 K-blocks, one FP32
    accumulator over all of K) and the first one past it (93 K-blocks, the fold
    kernel), FP32 output against the literal bound, with outlier channels."""
    rng = np.random.default_rng(K)
    M, N = 256, 512
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.001, 100.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    c = host64(run_dense(qa, sa, qb, sb, "128x128", "fp32"))
    check(c, *gemm.gemm_blockscaled_ref(qa, sa, qb, sb), "fp32", f"K={K}")


@pytest.mark.timeout(600)
def test_linear_trio_full_size():
    """Fprop / Dgrad / Wgrad of a 7168->2048 linear at 8192 tokens."""
    x, w, dy = workloads.linear_trio()
    rng = np.random.default_rng(43)
    # Fprop: Y = X . W^T   (M=8192 N=2048 K=7168)
    qx, sx = quant.quant_act_1x128(x)
    qw, sw = quant.quant_weight_128x128(w)
    c = run_dense(qx, sx, qw, sw, "128x128", "bf16")
    rows = sample_rows(8192, rng, 48)
    cr, s_abs = gemm.gemm_blockscaled_ref(qx, sx, qw, sw, rows=rows)
    check(host64(c[torch.from_numpy(rows).to(DEV)]), cr, s_abs, "bf16", "fprop")
    # Dgrad: dX = dY . W    (M=8192 N=7168 K=2048), B = transposed weight codes
    qd, sd = quant.quant_act_1x128(dy)
    qwt, swt = quant.quant_weight_128x128(w, transpose_out=True)
    c = run_dense(qd, sd, qwt, swt, "128x128", "bf16")
    cr, s_abs = gemm.gemm_blockscaled_ref(qd, sd, qwt, swt, rows=rows)
    check(host64(c[torch.from_numpy(rows).to(DEV)]), cr, s_abs, "bf16", "dgrad")
    # Wgrad: dW = dY^T . X  (M=2048 N=7168 K=8192), both operands 1x128 along tokens, FP32 out
    qdt, sdt = quant.quant_act_1x128_tokenwise(dy)
    qxt, sxt = quant.quant_act_1x128_tokenwise(x)
    c = run_dense(qdt, sdt, qxt, sxt, "1x128", "fp32")
    rows = sample_rows(2048, rng, 32)
    cr, s_abs = gemm.gemm_blockscaled_ref(qdt, sdt, qxt, sxt, "1x128", rows=rows)
    check(host64(c[torch.from_numpy(rows).to(DEV)]), cr, s_abs, "fp32", "wgrad")


_EXPERT_CACHE = {}


def _experts(kind, G, N, K):
    """Oracle-quantized expert weights (cached: the full-size layers are shared
    by the contiguous and masked tests)."""
    key = (kind, G, N, K)
    if key not in _EXPERT_CACHE:
        qs, ss = [], []
        for g in range(G):
            q, s = quant.quant_weight_128x128(workloads.expert_weight(kind, g, N, K))
            qs.append(q)
            ss.append(s)
        _EXPERT_CACHE.clear()
        _EXPERT_CACHE[key] = (np.stack(qs), np.stack(ss))
    return _EXPERT_CACHE[key]


def _layer(N, K):
    return "moe_gate_up" if (N, K) == (4096, 7168) else "moe_down"


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_contiguous_small_and_equal_to_dense(out):
    rng = np.random.default_rng(44)
    counts = np.array([5, 0, 300, 128, 1])
    off = workloads.pad_offsets(counts)
    G, N, K = 5, 256, 384
    a = workloads.activations(rng, int(off[-1]), K, 0.01, 100.0)
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = _experts("moe_contig", G, N, K)
    c = fp8.fp8_grouped_gemm_contiguous(dev(qa), dev(sa), dev(qb), dev(sb), dev(off.astype(np.int32)), OUT[out])
    rows, cr, s_abs = gemm.grouped_contiguous_ref(qa, sa, qb, sb, off)
    check(host64(c), cr, s_abs, out, "contiguous small")
    for g in range(G):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            cd = run_dense(qa[lo:hi], sa[:, lo:hi], qb[g], sb[g], "128x128", out)
            torch.cuda.synchronize()
            assert torch.equal(cd, c[lo:hi]), g


def test_contiguous_rows_outside_offsets_untouched():
    rng = np.random.default_rng(45)
    off = np.array([0, 128, 256], np.int32)          # M_total = 512: last two tiles belong to no group
    G, N, K = 2, 128, 256
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, 512, K))
    qb, sb = _experts("moe_contig", G, N, K)
    c = torch.full((512, N), 7.0, dtype=torch.float32, device=DEV)
    fp8.fp8_grouped_gemm_contiguous(dev(qa), dev(sa), dev(qb), dev(sb), dev(off), torch.float32, out=c)
    torch.cuda.synchronize()
    assert torch.all(c[256:] == 7.0)
    assert not torch.any(c[:256] == 7.0)


@pytest.mark.timeout(900)
def test_contiguous_moe_full_size():
    """32 experts, 65536 Zipf-routed rows padded per expert, K=7168 N=4096, BF16."""
    counts, off = workloads.moe_contig_layout()
    G, N, K = 32, 4096, 7168
    a = workloads.moe_contig_rows(counts, off, K)
    qa, sa = quant.quant_act_1x128(a)
    del a
    qb, sb = _experts(_layer(N, K), G, N, K)
    c = fp8.fp8_grouped_gemm_contiguous(dev(qa), dev(sa), dev(qb), dev(sb), dev(off.astype(np.int32)))
    rng = np.random.default_rng(46)
    rows = [np.arange(off[g], min(off[g] + 4, off[g + 1])) for g in range(G) if off[g + 1] > off[g]]
    rows += [np.arange(max(off[g], off[g + 1] - 4), off[g + 1]) for g in range(G) if off[g + 1] > off[g]]
    rows = np.unique(np.concatenate(rows + [rng.integers(0, int(off[-1]), 256)]))
    sel, cr, s_abs = gemm.grouped_contiguous_ref(qa, sa, qb, sb, off, rows=rows)
    check(host64(c[torch.from_numpy(sel).to(DEV)]), cr, s_abs, "bf16", "contiguous full")


def _masked_case(N, K, G=32, M_max=128):
    mm, a = workloads.moe_masked_inputs(N, K, G, M_max)
    qs, ss = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    return mm, np.stack(qs), np.stack(ss)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_masked_small_with_sentinel(out):
    G, M_max, N, K = 4, 96, 256, 256
    rng = np.random.default_rng(47)
    mm = np.array([1, 0, 96, 37], np.int32)
    a = np.stack([workloads.activations(rng, M_max, K, 0.01, 100.0) for _ in range(G)])
    qa, sa = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    qb, sb = _experts("moe_masked", G, N, K)
    c = torch.full((G, M_max, N), -3.0, dtype=OUT[out], device=DEV)
    fp8.fp8_grouped_gemm_masked(dev(qa), dev(sa), dev(qb), dev(sb), dev(mm), OUT[out], out=c)
    res = gemm.grouped_masked_ref(qa, sa, qb, sb, mm)
    ch = host64(c)
    for g in range(G):
        check(ch[g, :mm[g]], res[g][0], res[g][1], out, f"masked g={g}")
        assert np.all(ch[g, mm[g]:] == -3.0)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_masked_buffers_over_128_rows(out):
    """Masked buffers longer than 128 rows take the 256-row tile: ragged,
    empty and full experts, sentinel kept past masked_m."""
    G, M_max, N, K = 3, 300, 256, 384
    rng = np.random.default_rng(52)
    mm = np.array([300, 0, 129], np.int32)
    a = np.stack([workloads.activations(rng, M_max, K, 0.01, 100.0) for _ in range(G)])
    qa, sa = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    qb, sb = _experts("moe_masked", G, N, K)
    c = torch.full((G, M_max, N), -3.0, dtype=OUT[out], device=DEV)
    fp8.fp8_grouped_gemm_masked(dev(qa), dev(sa), dev(qb), dev(sb), dev(mm), OUT[out], out=c)
    res = gemm.grouped_masked_ref(qa, sa, qb, sb, mm)
    ch = host64(c)
    for g in range(G):
        check(ch[g, :mm[g]], res[g][0], res[g][1], out, f"masked>128 g={g}")
        assert np.all(ch[g, mm[g]:] == -3.0)


def test_masked_many_experts_every_row_once():
    """70 experts (140 expert/m-tile pairs: the kernel orders workgroups by the
    pairs' valid rows over several 64-pair chunks), counts covering 0, 1, 32,
    33, 64, 65, 127 and 128 rows: every valid row is computed, every other row
    keeps its sentinel."""
    G, M_max, N, K = 70, 128, 256, 256
    rng = np.random.default_rng(53)
    mm = rng.integers(0, M_max + 1, G).astype(np.int32)
    mm[:8] = [0, 1, 32, 33, 64, 65, 127, 128]
    a = np.stack([workloads.activations(rng, M_max, K, 0.01, 20.0) for _ in range(G)])
    qa, sa = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    qb, sb = _experts("moe_masked", G, N, K)
    for out in ("bf16", "fp32"):
        c = torch.full((G, M_max, N), -7.0, dtype=OUT[out], device=DEV)
        fp8.fp8_grouped_gemm_masked(dev(qa), dev(sa), dev(qb), dev(sb), dev(mm), OUT[out], out=c)
        res = gemm.grouped_masked_ref(qa, sa, qb, sb, mm)
        ch = host64(c)
        for g in range(G):
            check(ch[g, :mm[g]], res[g][0], res[g][1], out, f"many experts g={g} rows={mm[g]}")
            assert np.all(ch[g, mm[g]:] == -7.0), g


# (G, M_max, N, K): the persistent decode kernel on 256-wide items (16 pairs:
# items grouped per XCD when the live pairs allow), the 256 x 256 tile
# (M_max > 128: 8 pairs), the fold decode tile (N = 128 mod 256: 16 pairs),
# 12 pairs, and 512-wide items with a last half K-block (K = 192, 320)
@pytest.mark.parametrize("G,M_max,N,K", [(8, 128, 768, 384), (4, 300, 512, 256), (8, 96, 384, 256),
                                         (6, 128, 512, 256), (8, 128, 1024, 192), (5, 64, 512, 320)])
def test_masked_equals_dense_per_expert(G, M_max, N, K):
    """Every expert's valid rows of the masked GEMM equal, bit for bit, the
    dense GEMM of those rows with that expert's weights: where a tile runs and
    in which order cannot change its bits (the arithmetic per output is the
    same in every kernel of the exact engine).  Also inside the oracle's bound;
    rows past masked_m keep their sentinel."""
    rng = np.random.default_rng(G * 1000 + M_max + N + K)
    mm = rng.integers(0, M_max + 1, G).astype(np.int32)
    mm[:3] = [M_max, 0, 1]
    a = np.stack([workloads.activations(rng, M_max, K, 0.01, 50.0) for _ in range(G)])
    qa, sa = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    qs, ss = zip(*[quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)])
    qb, sb = np.stack(qs), np.stack(ss)
    c = torch.full((G, M_max, N), -5.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_masked(dev(qa), dev(sa), dev(qb), dev(sb), dev(mm), torch.bfloat16, out=c)
    torch.cuda.synchronize()
    res = gemm.grouped_masked_ref(qa, sa, qb, sb, mm)
    ch = c.cpu()
    for g in range(G):
        m = int(mm[g])
        assert torch.all(ch[g, m:] == -5.0), g
        if m == 0:
            continue
        cd = run_dense(qa[g, :m], np.ascontiguousarray(sa[g][:, :m]), qb[g], sb[g], "128x128", "bf16").cpu()
        assert torch.equal(cd.view(torch.int16), ch[g, :m].view(torch.int16)), f"expert {g}"
        check(ch[g, :m].double().numpy(), res[g][0], res[g][1], "bf16", f"masked g={g}")


def test_masked_counts_out_of_range_are_clamped():
    """masked_m values are clamped to [0, M_max] on the device: a negative
    count computes and writes nothing, one above M_max computes every row."""
    rng = np.random.default_rng(77)
    G, M_max, N, K = 4, 64, 256, 256
    mm_dev = np.array([-5, M_max + 7, 3, -1], np.int32)
    mm = np.clip(mm_dev, 0, M_max)
    a = np.stack([workloads.activations(rng, M_max, K, 0.01, 50.0) for _ in range(G)])
    qa, sa = zip(*[quant.quant_act_1x128(a[g]) for g in range(G)])
    qa, sa = np.stack(qa), np.stack(sa)
    qs, ss = zip(*[quant.quant_weight_128x128(workloads.weights(rng, N, K)) for _ in range(G)])
    qb, sb = np.stack(qs), np.stack(ss)
    for out in ("bf16", "fp32"):
        c = torch.full((G, M_max, N), 9.0, dtype=OUT[out], device=DEV)
        fp8.fp8_grouped_gemm_masked(dev(qa), dev(sa), dev(qb), dev(sb), dev(mm_dev), OUT[out], out=c)
        ch = host64(c)
        res = gemm.grouped_masked_ref(qa, sa, qb, sb, mm)
        for g in range(G):
            assert np.all(ch[g, mm[g]:] == 9.0), (out, g)
            if mm[g]:
                check(ch[g, :mm[g]], res[g][0], res[g][1], out, f"clamped g={g}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)])
def test_masked_moe_full_size(N, K):
    """32 experts, 128-row buffers, valid rows U{1..64}: sampled valid rows per
    expert against the oracle; every row past masked_m keeps its sentinel."""
    G, M_max = 32, 128
    mm, qa, sa = _masked_case(N, K, G, M_max)
    qb, sb = _experts(_layer(N, K), G, N, K)
    c = torch.full((G, M_max, N), 5.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_masked(dev(qa), dev(sa), dev(qb), dev(sb), dev(mm.astype(np.int32)), out=c)
    torch.cuda.synchronize()
    rng = np.random.default_rng(48)
    for g in range(G):
        m = int(mm[g])
        assert bool(torch.all(c[g, m:] == 5.0)), g
        rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 4)]))
        cr, s_abs = gemm.gemm_blockscaled_ref(qa[g], sa[g], qb[g], sb[g], rows=rows)
        check(host64(c[g][torch.from_numpy(rows).to(DEV)]), cr, s_abs, "bf16", f"masked full g={g}")


# ---------------------------------------------------------------------------
# The FP8-MFMA engine (fp8_gemm_blockscaled_fp8mfma).  gfx950's FP8 MFMA
# adds its products in groups of eight consecutive K and truncates each to 13
# fractional bits below the group's largest exponent (measured, see the design
# notes), so each group can lose up to 7 * 2^-13 of its largest product, and
# twice that when the largest product involves a subnormal code.  The engine is
# therefore held to u = 2^-9 instead of 2^-14.
U_FP8MFMA = 2.0 ** -9


def run_fp8mfma(qa, sa, qb, sb, kind, out):
    return fp8.fp8_gemm_blockscaled_fp8mfma(dev(qa), dev(sa), dev(qb), dev(sb), BS[kind], OUT[out])


def test_fp8mfma_in_group_truncation_model():
    """448*448 + 127 * (1 * 0.5): the seven 0.5-products that share the big
    product's group of eight are truncated away (grid 2^(16-13) = 8)."""
    a, b, exp = gemm_hand_case()
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    c = host64(run_fp8mfma(qa, sa, qb, sb, "128x128", "fp32"))
    assert c[0, 0] == 200704.0 + 120 * 0.5
    assert np.all(c[0, 1:] == exp[("fp32", "n_other")])


@pytest.mark.parametrize("M,N,K", [(17, 256, 256), (130, 384, 1024), (300, 512, 2048)])
@pytest.mark.parametrize("kind", ["128x128", "1x128"])
def test_fp8mfma_engine_bound(M, N, K, kind):
    rng = np.random.default_rng(M + N + K)
    a = workloads.activations(rng, M, K, 0.01, 50.0)
    b = workloads.weights(rng, N, K) if kind == "128x128" else workloads.activations(rng, N, K, 0.0, 1.0, 1e-3)
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant_b(b, kind)
    c = host64(run_fp8mfma(qa, sa, qb, sb, kind, "fp32"))
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, kind)
    assert np.all(np.abs(c - c_ref) <= U_FP8MFMA * s_abs)


# The FP8-MFMA engine on the MX kernel's tiling (dense, 128x128-scaled B,
# N % 256 == 0, K % 64 == 0): the scales' powers of two ride in the scaled
# MFMA's E8M0 bytes, their mantissa parts in the accumulator's unit.

def _check_fp8mfma(c, c_ref, s_abs, out, what):
    lim = U_FP8MFMA * s_abs if out == "fp32" else U_FP8MFMA * s_abs * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(c_ref)
    err = np.abs(c - c_ref)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, f"{what}: {len(bad)} outside, max err/bound {np.max(err / np.maximum(lim, 1e-300)):.3g}"


def test_fp8mfma_tiled_in_group_truncation_model():
    """The hand case on 256 output columns (the MX tiling): C[0][0] keeps the
    in-group truncation of the instruction, 448*448 + 120 * 0.5, and the
    other columns of the first 128-column block are exact."""
    a, b128, exp = gemm_hand_case()
    b = np.concatenate([b128, np.full((128, 128), 0.25, np.float32)])
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    c = host64(run_fp8mfma(qa, sa, qb, sb, "128x128", "fp32"))
    assert c[0, 0] == 200704.0 + 120 * 0.5
    assert np.all(c[0, 1:128] == exp[("fp32", "n_other")])
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128")
    _check_fp8mfma(c[:, 128:], c_ref[:, 128:], s_abs[:, 128:], "fp32", "hand case, second block")


@pytest.mark.parametrize("M,N,K", [(1, 256, 64), (257, 512, 1088), (300, 768, 2112)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_fp8mfma_tiled_bound(M, N, K, out):
    """Ragged M, a last K-block of 64 (K = 1088, 2112), scales spread over many
    binades with a subnormal one, and zero scales over nonzero codes (row 5's
    all zero: its outputs must be exactly 0)."""
    rng = np.random.default_rng(M + N + K + (out == "fp32"))
    qa, sa = quant.quant_act_1x128(workloads.activations(rng, M, K, 0.01, 50.0))
    qb, sb = quant.quant_weight_128x128(workloads.weights(rng, N, K))
    sa = (sa * np.exp2(rng.integers(-40, 41, sa.shape))).astype(np.float32)
    sb = (sb * np.exp2(rng.integers(-20, 21, sb.shape))).astype(np.float32)
    sa[rng.random(sa.shape) < 0.1] = 0.0
    sb[rng.random(sb.shape) < 0.1] = 0.0
    if M > 5:
        sa[:, 5] = 0.0
        sa[-1, 3] = np.float32(2.0 ** -140)
    c = host64(run_fp8mfma(qa, sa, qb, sb, "128x128", out))
    c_ref, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, "128x128")
    assert np.all(np.isfinite(c))
    _check_fp8mfma(c, c_ref, s_abs, out, f"fp8mfma tiled {M}x{N}x{K} {out}")
    if M > 5:
        assert np.all(c[5] == 0.0)


@pytest.mark.timeout(600)
def test_fp8mfma_full_size_dense_fprop():
    """The 4096x7168x2048 workload on the FP8-MFMA engine: sampled rows within
    its bound."""
    x, w = workloads.dense_fprop()
    qa, sa = quant.quant_act_1x128(x)
    qb, sb = quant.quant_weight_128x128(w)
    c = run_fp8mfma(qa, sa, qb, sb, "128x128", "bf16")
    rows = sample_rows(4096, np.random.default_rng(52), 48)
    cr, s_abs = gemm.gemm_blockscaled_ref(qa, sa, qb, sb, rows=rows)
    _check_fp8mfma(host64(c[torch.from_numpy(rows).to(DEV)]), cr, s_abs, "bf16", "fp8mfma full size")
