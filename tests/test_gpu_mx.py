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


# ---------------------------------------------------------------------------
# The MX GEMM in the MoE layouts.  Each expert's rows must be exactly what the
# dense MX call gives for that expert's operands (same arithmetic, same tile
# origin), and within the MX bound of the oracle.

def _mx_experts(rng, G, N, K):
    qs, es = zip(*[mx.quant_mx_1x32(workloads.weights(rng, N, K)) for _ in range(G)])
    return np.stack(qs), np.stack(es)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_mx_contiguous_equals_dense_per_group(out):
    """Groups of 256, 0, 128 and 384 rows (tiles of 256 rows straddle a group
    end), N = 512, K = 320 (five 64-K stages)."""
    rng = np.random.default_rng(91)
    off = np.array([0, 256, 256, 384, 768], np.int32)
    G, N, K = 4, 512, 320
    qa, ea = mx.quant_mx_1x32(workloads.activations(rng, int(off[-1]), K, 0.01, 50.0))
    qb, eb = _mx_experts(rng, G, N, K)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    c = fp8.fp8_grouped_gemm_contiguous_mx(dev(qa), dev(ea), dev(qb), dev(eb), dev(off), od)
    ch = c.float().cpu().numpy().astype(np.float64)
    for g in range(G):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        cd = fp8.fp8_gemm_mx(dev(qa[lo:hi]), dev(ea[:, lo:hi]), dev(qb[g]), dev(eb[g]), od)
        torch.cuda.synchronize()
        assert torch.equal(cd, c[lo:hi]), g
        _check(ch[lo:hi], mx.dequant_mx(qa[lo:hi], ea[:, lo:hi]), mx.dequant_mx(qb[g], eb[g]), out,
               f"mx contiguous g={g} {out}")


def test_mx_contiguous_rows_outside_offsets_untouched():
    rng = np.random.default_rng(92)
    off = np.array([0, 128, 256], np.int32)          # M_total = 512: rows 256.. belong to no group
    G, N, K = 2, 256, 128
    qa, ea = mx.quant_mx_1x32(workloads.activations(rng, 512, K))
    qb, eb = _mx_experts(rng, G, N, K)
    c = torch.full((512, N), 7.0, dtype=torch.float32, device=DEV)
    fp8.fp8_grouped_gemm_contiguous_mx(dev(qa), dev(ea), dev(qb), dev(eb), dev(off), torch.float32, out=c)
    torch.cuda.synchronize()
    assert torch.all(c[256:] == 7.0)
    assert not torch.any(c[:256] == 7.0)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_mx_masked_equals_dense_per_expert(out):
    """Buffers of 320 rows (two 256-row m-tiles), valid counts 0, 1, 257, 320,
    77 and two out-of-range values that the device clamps (-3 -> 0, 999 -> 320);
    rows past the count keep their sentinel."""
    rng = np.random.default_rng(93)
    G, M_max, N, K = 7, 320, 512, 192
    mm_dev = np.array([0, 1, 257, 320, 77, -3, 999], np.int32)
    mm = np.clip(mm_dev, 0, M_max)
    qa, ea = zip(*[mx.quant_mx_1x32(workloads.activations(rng, M_max, K, 0.01, 50.0)) for _ in range(G)])
    qa, ea = np.stack(qa), np.stack(ea)
    qb, eb = _mx_experts(rng, G, N, K)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    c = torch.full((G, M_max, N), 9.0, dtype=od, device=DEV)
    fp8.fp8_grouped_gemm_masked_mx(dev(qa), dev(ea), dev(qb), dev(eb), dev(mm_dev), od, out=c)
    torch.cuda.synchronize()
    for g in range(G):
        m = int(mm[g])
        assert bool(torch.all(c[g, m:] == 9.0)), g
        if m == 0:
            continue
        cd = fp8.fp8_gemm_mx(dev(qa[g]), dev(ea[g]), dev(qb[g]), dev(eb[g]), od)
        torch.cuda.synchronize()
        assert torch.equal(cd[:m], c[g, :m]), g
        _check(c[g, :m].float().cpu().numpy().astype(np.float64), mx.dequant_mx(qa[g], ea[g])[:m],
               mx.dequant_mx(qb[g], eb[g]), out, f"mx masked g={g} {out}")


@pytest.mark.timeout(900)
def test_mx_masked_decode_full_size():
    """The masked decode workload's down projection (32 experts, 128-row
    buffers, valid rows U{1..64}, K = 2048, N = 7168), MX-quantized by the
    oracle: sampled valid rows of every expert within the MX bound, every row
    past masked_m keeps its sentinel."""
    G, M_max, N, K = 32, 128, 7168, 2048
    mm, a = workloads.moe_masked_inputs(N, K, G, M_max)
    qa, ea = zip(*[mx.quant_mx_1x32(a[g]) for g in range(G)])
    qa, ea = np.stack(qa), np.stack(ea)
    del a
    qb, eb = zip(*[mx.quant_mx_1x32(workloads.expert_weight("moe_down", g, N, K)) for g in range(G)])
    qb, eb = np.stack(qb), np.stack(eb)
    c = torch.full((G, M_max, N), 5.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_masked_mx(dev(qa), dev(ea), dev(qb), dev(eb), dev(mm.astype(np.int32)), out=c)
    torch.cuda.synchronize()
    rng = np.random.default_rng(94)
    for g in range(G):
        m = int(mm[g])
        assert bool(torch.all(c[g, m:] == 5.0)), g
        rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 3)]))
        cg = c[g][torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
        _check(cg, mx.dequant_mx(qa[g], ea[g])[rows], mx.dequant_mx(qb[g], eb[g]), "bf16", f"mx masked full g={g}")


# ---------------------------------------------------------------------------
# MX operands blocked along the rows (tokens for Wgrad, output features for
# the Dgrad weight): the transposed quantizer and the MX trio of a Linear.

def _inputs_t(rng, M, K):
    x = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-6, 6, size=(1, K)))).astype(np.float32)
    if M >= 96 and K > 2:
        x[:32, 0] = 0.0
        x[5, 0] = -0.0
        x[32:64, 1] = np.float32(1.9)                           # saturation
        x[64:96, 2] = np.float32(2.0 ** -130) * np.arange(32)   # subnormal block: scale clamps
    return x


@pytest.mark.parametrize("M,K", [(32, 1), (96, 70), (128, 64), (160, 300), (4096, 33)])
def test_quant_mx_transposed_bit_exact(M, K):
    x = _inputs_t(np.random.default_rng(M + 5 * K), M, K)
    q, e = fp8.fp8_quant_mx_1x32_transposed(dev(x))
    oq, oe = mx.quant_mx_1x32_transposed(x)
    assert np.array_equal(host(e), oe)
    bad = np.argwhere(host(q) != oq)
    assert bad.size == 0, bad[:5].tolist()


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_mx_linear_trio_small(out):
    """Fprop, Dgrad and Wgrad of a 512 -> 256 Linear at 192 tokens, every
    operand MX-quantized by the oracle along its GEMM's contraction; the GPU
    quantizers give the same bytes."""
    rng = np.random.default_rng(95)
    T, IN, OUT = 192, 512, 256
    x = workloads.activations(rng, T, IN, 0.01, 50.0)
    w = workloads.weights(rng, OUT, IN)
    dy = workloads.activations(rng, T, OUT, sigma=1e-3)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    qx, ex = mx.quant_mx_1x32(x)
    qw, ew = mx.quant_mx_1x32(w)
    qd, ed = mx.quant_mx_1x32(dy)
    qwt, ewt = mx.quant_mx_1x32_transposed(w)       # W^T [IN][OUT], blocks along OUT
    qdt, edt = mx.quant_mx_1x32_transposed(dy)      # dY^T [OUT][T], blocks along tokens
    qxt, ext = mx.quant_mx_1x32_transposed(x)       # X^T [IN][T]
    for src, (oq, oe) in ((w, (qwt, ewt)), (dy, (qdt, edt)), (x, (qxt, ext))):
        gq, ge = fp8.fp8_quant_mx_1x32_transposed(dev(src))
        assert np.array_equal(host(gq), oq) and np.array_equal(host(ge), oe)
    for name, (qa, ea, qb, eb) in (("fprop", (qx, ex, qw, ew)), ("dgrad", (qd, ed, qwt, ewt)),
                                   ("wgrad", (qdt, edt, qxt, ext))):
        c = fp8.fp8_gemm_mx(dev(qa), dev(ea), dev(qb), dev(eb), od)
        _check(c.float().cpu().numpy().astype(np.float64), mx.dequant_mx(qa, ea), mx.dequant_mx(qb, eb), out,
               f"mx trio {name} {out}")


@pytest.mark.timeout(900)
def test_mx_wgrad_full_size():
    """dW = dY^T . X of the 7168 -> 2048 Linear at 8192 tokens (M = 2048,
    N = 7168, K = 8192), both operands MX along tokens: the GPU quantizer's
    bytes equal the oracle's, and sampled rows of the FP32 dW are within the
    MX bound."""
    x, _, dy = workloads.linear_trio()
    qdt, edt = mx.quant_mx_1x32_transposed(dy)
    qxt, ext = mx.quant_mx_1x32_transposed(x)
    gq, ge = fp8.fp8_quant_mx_1x32_transposed(dev(x))
    assert np.array_equal(host(ge), ext) and np.array_equal(host(gq), qxt)
    del gq, ge
    c = fp8.fp8_gemm_mx(dev(qdt), dev(edt), dev(qxt), dev(ext), torch.float32)
    rows = np.unique(np.concatenate([np.random.default_rng(96).choice(2048, 24, replace=False), [0, 2047]]))
    torch.cuda.synchronize()
    cg = c[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    _check(cg, mx.dequant_mx(qdt, edt)[rows], mx.dequant_mx(qxt, ext), "fp32", "mx wgrad full size")


# The MX masked GEMM on decode-tiled weights: the persistent register-stream
# kernel, bit for bit the plain-weight MX call.

@pytest.mark.parametrize("G,M_max,N,K,out", [(8, 128, 512, 384, "bf16"), (5, 64, 768, 320, "fp32"),
                                             (4, 100, 256, 64, "bf16"), (8, 96, 1024, 1152, "fp32"),
                                             (8, 128, 1792, 448, "bf16"), (4, 128, 3584, 192, "fp32")])
def test_mx_masked_tiled_equals_plain(G, M_max, N, K, out):
    """Ragged valid counts (M_max, 0, 1, 33, ...), K with a half K-block past
    the last whole one, items of 256, 448 and 512 columns; rows past masked_m
    keep their sentinel; the valid rows are within the MX bound of the oracle."""
    from oracle import layout
    if M_max % 4:
        M_max += 4 - M_max % 4
    rng = np.random.default_rng(G * 100 + M_max + N + K + 7)
    mm = rng.integers(0, M_max + 1, G).astype(np.int32)
    mm[:4] = [M_max, 0, 1, 33]
    qa, ea = zip(*[mx.quant_mx_1x32(workloads.activations(rng, M_max, K, 0.01, 50.0)) for _ in range(G)])
    qa, ea = np.stack(qa), np.stack(ea)
    qb, eb = _mx_experts(rng, G, N, K)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    args = [dev(qa), dev(ea)]
    c_t = torch.full((G, M_max, N), -9.0, dtype=od, device=DEV)
    fp8.fp8_grouped_gemm_masked_tiled_mx(*args, dev(layout.tile_weights_decode(qb)), dev(eb), dev(mm), od, out=c_t)
    c_p = torch.full((G, M_max, N), -9.0, dtype=od, device=DEV)
    fp8.fp8_grouped_gemm_masked_mx(*args, dev(qb), dev(eb), dev(mm), od, out=c_p)
    torch.cuda.synchronize()
    assert torch.equal(c_t.view(torch.int16 if out == "bf16" else torch.int32),
                       c_p.view(torch.int16 if out == "bf16" else torch.int32)), "the tiled layout changed the result"
    ch = c_t.float().cpu().numpy().astype(np.float64)
    for g in range(G):
        m = int(mm[g])
        assert np.all(ch[g, m:] == -9.0), g
        if m:
            _check(ch[g, :m], mx.dequant_mx(qa[g], ea[g])[:m], mx.dequant_mx(qb[g], eb[g]), out, f"mx tiled g={g}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)])
def test_mx_masked_tiled_full_size_equals_plain(N, K):
    """The masked decode shapes (32 experts, 128-row buffers, rows U{1..64}),
    MX-quantized and tiled by the GPU: the same bits as the plain-weight MX
    call (whose oracle parity at this size is test_mx_masked_decode_full_size)."""
    G, M_max = 32, 128
    g = torch.Generator(device=DEV).manual_seed(N + 5 * K)
    qa = torch.empty((G, M_max, K), dtype=torch.uint8, device=DEV)
    ea = torch.empty((G, K // 32, M_max), dtype=torch.uint8, device=DEV)
    qb = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    eb = torch.empty((G, K // 32, N), dtype=torch.uint8, device=DEV)
    for e in range(G):
        fp8.fp8_quant_mx_1x32(torch.randn((M_max, K), generator=g, device=DEV), q=qa[e], e=ea[e])
        fp8.fp8_quant_mx_1x32(torch.randn((N, K), generator=g, device=DEV) * 0.02, q=qb[e], e=eb[e])
    mm = torch.randint(1, 65, (G,), generator=g, device=DEV, dtype=torch.int32)
    c_t = torch.full((G, M_max, N), 5.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_masked_tiled_mx(qa, ea, fp8.fp8_tile_weights_decode(qb), eb, mm, out=c_t)
    c_p = torch.full((G, M_max, N), 5.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_grouped_gemm_masked_mx(qa, ea, qb, eb, mm, out=c_p)
    torch.cuda.synchronize()
    assert torch.equal(c_t.view(torch.int16), c_p.view(torch.int16))
