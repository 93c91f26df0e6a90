"""GPU parity of the quantizers against the CPU oracle: codes and scales must be
bit-identical.  All calls go through the C ABI (ctypes binding)."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amd as fp8
from oracle import e4m3, quant
from tests.goldens import quant_tile_cases
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_same(gq, gs, oq, os_, what):
    gq, gs = host(gq), host(gs)
    bad = np.argwhere(gq != oq)
    assert bad.size == 0, f"{what}: {len(bad)} code mismatches, first at {bad[:3].tolist()}"
    assert np.array_equal(gs.view(np.uint32), np.asarray(os_, np.float32).view(np.uint32)), f"{what}: scales differ"


def test_golden_tiles_on_gpu():
    for name, tile, scale, codes in quant_tile_cases():
        x = np.tile(tile, (3, 2))
        q, s = fp8.fp8_quant_act_1x128(dev(x))
        q, s = host(q), host(s)
        assert np.all(s.view(np.uint32) == np.float32(scale).view(np.uint32)), name
        for r in range(3):
            for kb in range(2):
                assert np.array_equal(q[r, kb * 128:(kb + 1) * 128], codes), name


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (128, 512), (257, 384), (1000, 1024)])
def test_act_rowwise_random(M, K):
    rng = np.random.default_rng(M * 7 + K)
    x = workloads.activations(rng, M, K, 0.01, 100.0)
    q, s = fp8.fp8_quant_act_1x128(dev(x))
    assert_same(q, s, *quant.quant_act_1x128(x), f"rowwise {M}x{K}")


@pytest.mark.parametrize("M,K", [(128, 1), (128, 64), (256, 100), (384, 517), (128, 2048)])
def test_act_tokenwise_random(M, K):
    rng = np.random.default_rng(M + 13 * K)
    x = workloads.activations(rng, M, K, 0.01, 100.0)
    q, s = fp8.fp8_quant_act_1x128(dev(x), transpose_out=True)
    assert_same(q, s, *quant.quant_act_1x128_tokenwise(x), f"tokenwise {M}x{K}")


@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (1024, 512)])
@pytest.mark.parametrize("transpose", [False, True])
def test_weight_random(N, K, transpose):
    rng = np.random.default_rng(N + K)
    w = workloads.weights(rng, N, K)
    w[5, 7] = 3.0                                      # one block with an outlier
    q, s = fp8.fp8_quant_weight_128x128(dev(w), transpose_out=transpose)
    assert_same(q, s, *quant.quant_weight_128x128(w, transpose_out=transpose), f"weight {N}x{K} T={transpose}")


def test_special_tiles():
    """Zero tiles, -0, fp32 subnormals, amax whose scale underflows, ties."""
    x = np.zeros((6, 256), np.float32)
    x[0, 3] = -0.0
    x[1, :128] = np.float32(1e-40) * np.arange(128, dtype=np.float32)     # subnormal amax
    x[2, 0] = np.float32(2e-45)                                            # scale underflows to 0
    x[2, 1] = -np.float32(1.4e-45)
    x[3, :128] = np.linspace(-448, 448, 128, dtype=np.float32)
    x[4, 128:] = np.float32(3.4e38) * np.linspace(-1, 1, 128, dtype=np.float32)
    x[5, :] = np.float32(2.0 ** -10) * np.arange(256) / 7
    q, s = fp8.fp8_quant_act_1x128(dev(x))
    assert_same(q, s, *quant.quant_act_1x128(x), "special tiles")
    xt = np.ascontiguousarray(np.tile(x, (22, 1))[:128])
    q, s = fp8.fp8_quant_act_1x128(dev(xt), transpose_out=True)
    assert_same(q, s, *quant.quant_act_1x128_tokenwise(xt), "special tiles, token-wise")


def _binade(e):
    base = np.uint32((e + 127) << 23)
    return (np.arange(1 << 23, dtype=np.uint32) + base).view(np.float32)


def test_exhaustive_encoder_through_unit_scale_tiles():
    """Every fp32 with exponent -11..8 up to 448 (both signs) goes through the
    GPU quantizer in a tile whose max-abs is 448, so the scale is exactly 1 and
    the code is the plain E4M3 encoding of the value: compared with the
    oracle's encoder on all of them."""
    for e in range(-11, 9):
        v = _binade(e)
        v = v[v <= 448.0]
        n_tiles = (v.size + 126) // 127
        x = np.zeros((n_tiles, 128), np.float32)
        x[:, 0] = 448.0
        flat = x[:, 1:].reshape(-1)
        flat[:v.size] = v
        x[:, 1:] = flat.reshape(n_tiles, 127)
        x[1::2] *= -1.0
        q, s = fp8.fp8_quant_act_1x128(dev(x))
        q, s = host(q), host(s)
        assert np.all(s == 1.0), e
        exp = e4m3.encode(x)
        bad = np.argwhere(q != exp)
        assert bad.size == 0, (e, bad[:3].tolist(), x[tuple(bad[0])] if bad.size else None)


def test_full_size_quantizers_dense_fprop():
    """The 4096x2048 activations and 7168x2048 weights of the dense Fprop workload."""
    x, w = workloads.dense_fprop()
    q, s = fp8.fp8_quant_act_1x128(dev(x))
    assert_same(q, s, *quant.quant_act_1x128(x), "dense_fprop activations")
    q, s = fp8.fp8_quant_weight_128x128(dev(w))
    assert_same(q, s, *quant.quant_weight_128x128(w), "dense_fprop weights")


def test_full_size_quantizers_linear_trio():
    x, w, dy = workloads.linear_trio()
    for name, arr in (("X", x), ("dY", dy)):
        q, s = fp8.fp8_quant_act_1x128(dev(arr))
        assert_same(q, s, *quant.quant_act_1x128(arr), f"trio {name} rowwise")
        q, s = fp8.fp8_quant_act_1x128(dev(arr), transpose_out=True)
        assert_same(q, s, *quant.quant_act_1x128_tokenwise(arr), f"trio {name} token-wise")
    for t in (False, True):
        q, s = fp8.fp8_quant_weight_128x128(dev(w), transpose_out=t)
        assert_same(q, s, *quant.quant_weight_128x128(w, transpose_out=t), f"trio W T={t}")


# ---------------------------------------------------------------------------
# bf16 inputs: the entry points widen each bf16 exactly to fp32, so their codes
# and scales must equal the oracle's on the widened values.  Inputs are made
# bf16-representable by clearing the low 16 bits of fp32 values.

def bf16_pair(x):
    bits = np.ascontiguousarray(x, np.float32).view(np.uint32)
    widened = (bits & np.uint32(0xFFFF0000)).view(np.float32)
    top = (bits >> np.uint32(16)).astype(np.uint16)
    return torch.from_numpy(top).to(DEV).view(torch.bfloat16), widened


@pytest.mark.parametrize("M,K", [(1, 128), (5, 384), (257, 1024)])
def test_bf16_act_rowwise(M, K):
    rng = np.random.default_rng(3 * M + K)
    xb, x = bf16_pair(workloads.activations(rng, M, K, 0.01, 100.0))
    q, s = fp8.fp8_quant_act_1x128_bf16(xb)
    assert_same(q, s, *quant.quant_act_1x128(x), f"bf16 rowwise {M}x{K}")


@pytest.mark.parametrize("M,K", [(128, 1), (128, 6), (256, 100), (384, 516), (128, 2048)])
def test_bf16_act_tokenwise(M, K):
    rng = np.random.default_rng(5 * M + K)
    xb, x = bf16_pair(workloads.activations(rng, M, K, 0.01, 100.0))
    q, s = fp8.fp8_quant_act_1x128_bf16(xb, transpose_out=True)
    assert_same(q, s, *quant.quant_act_1x128_tokenwise(x), f"bf16 tokenwise {M}x{K}")


@pytest.mark.parametrize("N,K", [(128, 128), (384, 256)])
@pytest.mark.parametrize("transpose", [False, True])
def test_bf16_weight(N, K, transpose):
    rng = np.random.default_rng(N * 3 + K)
    w = workloads.weights(rng, N, K)
    w[N - 1, 9] = -2.5
    wb, w = bf16_pair(w)
    q, s = fp8.fp8_quant_weight_128x128_bf16(wb, transpose_out=transpose)
    assert_same(q, s, *quant.quant_weight_128x128(w, transpose_out=transpose), f"bf16 weight {N}x{K} T={transpose}")


def test_bf16_special_tiles():
    """bf16 subnormals, -0, a scale that underflows, the largest bf16 values."""
    x = np.zeros((6, 256), np.float32)
    x[0, 3] = -0.0
    x[1, :128] = np.float32(2.0 ** -133) * np.arange(128, dtype=np.float32)
    x[2, 0] = np.float32(2.0 ** -133)
    x[3, :128] = np.linspace(-448, 448, 128, dtype=np.float32)
    x[4, 128:] = np.float32(3.38e38) * np.linspace(-1, 1, 128, dtype=np.float32)
    x[5, :] = np.float32(2.0 ** -10) * np.arange(256) / 7
    xb, xw = bf16_pair(x)
    q, s = fp8.fp8_quant_act_1x128_bf16(xb)
    assert_same(q, s, *quant.quant_act_1x128(xw), "bf16 special tiles")
    xb, xw = bf16_pair(np.tile(x, (22, 1))[:128])
    q, s = fp8.fp8_quant_act_1x128_bf16(xb, transpose_out=True)
    assert_same(q, s, *quant.quant_act_1x128_tokenwise(xw), "bf16 special tiles, token-wise")
    wb, ww = bf16_pair(np.tile(x[:, :128], (22, 1))[:128])
    for t in (False, True):
        q, s = fp8.fp8_quant_weight_128x128_bf16(wb, transpose_out=t)
        assert_same(q, s, *quant.quant_weight_128x128(ww, transpose_out=t), f"bf16 special weight T={t}")


def test_bf16_full_size_linear_trio():
    x, w, dy = workloads.linear_trio()
    for name, arr in (("X", x), ("dY", dy)):
        ab, aw = bf16_pair(arr)
        q, s = fp8.fp8_quant_act_1x128_bf16(ab)
        assert_same(q, s, *quant.quant_act_1x128(aw), f"bf16 trio {name} rowwise")
        q, s = fp8.fp8_quant_act_1x128_bf16(ab, transpose_out=True)
        assert_same(q, s, *quant.quant_act_1x128_tokenwise(aw), f"bf16 trio {name} token-wise")
    wb, ww = bf16_pair(w)
    for t in (False, True):
        q, s = fp8.fp8_quant_weight_128x128_bf16(wb, transpose_out=t)
        assert_same(q, s, *quant.quant_weight_128x128(ww, transpose_out=t), f"bf16 trio W T={t}")


# ---------------------------------------------------------------------------
# FP8 activation cache -> token-wise operand: bit-exact against the oracle.

def _cache(rng, R, K):
    q = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01                          # no NaN codes
    s = np.exp(rng.uniform(np.log(1e-8), np.log(1e4), size=(K // 128, R))).astype(np.float32)
    s[0, 1] = 0.0
    s[-1, 2] = np.float32(7e-41)
    return q, s


@pytest.mark.parametrize("M,K", [(128, 128), (256, 384), (384, 1024)])
def test_requant_random(M, K):
    rng = np.random.default_rng(M * 3 + K * 5)
    q, s = _cache(rng, M, K)
    qt, st = fp8.fp8_requant_act_tokenwise(dev(q), dev(s))
    assert_same(qt, st, *quant.requant_act_tokenwise(q, s), f"requant {M}x{K}")


def test_requant_every_code():
    """All 254 non-NaN codes, each in every token position class, under unit,
    power-of-two and general row scales."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    q = np.resize(codes, (256, 512)).astype(np.uint8)
    q[1::2] = np.roll(q[1::2], 37, axis=1)
    s = np.ones((4, 256), np.float32)
    s[1] = 2.0 ** -7
    s[2] = np.float32(1.0 / 3.0)
    s[3] = np.linspace(1e-3, 10, 256, dtype=np.float32)
    qt, st = fp8.fp8_requant_act_tokenwise(dev(q), dev(s))
    assert_same(qt, st, *quant.requant_act_tokenwise(q, s), "requant every code")


def test_requant_full_size_linear_trio():
    """The Wgrad operand of the 8192x7168 activations, from their rowwise cache."""
    x, _, _ = workloads.linear_trio()
    q, s = quant.quant_act_1x128(x)
    qt, st = fp8.fp8_requant_act_tokenwise(dev(q), dev(s))
    assert_same(qt, st, *quant.requant_act_tokenwise(q, s), "requant trio X")


# ---------------------------------------------------------------------------
# Both Fprop operands in one launch: byte for byte the two separate calls, and
# the oracle's codes and scales.
def _bf16_bits(a):
    """float32 array -> the bf16 tensor of its upper halves (exact widening back)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to(torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(37, 272, 1040), (256, 512, 384), (1, 16, 16), (0, 144, 256), (96, 0, 256)])
@pytest.mark.parametrize("xb,wb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_fprop_operands_match_separate_calls_and_oracle(M, N, K, xb, wb):
    rng = np.random.default_rng(M + 3 * N + 7 * K + 11 * xb + 13 * wb)
    x = workloads.activations(rng, max(M, 1), K, 0.01, 50.0)[:M]
    w = workloads.weights(rng, max(N, 1), K)[:N]
    xt = _bf16_bits(x).to(DEV) if xb else dev(x)
    wt = _bf16_bits(w).to(DEV) if wb else dev(w)
    qa, sa, qb, sb = fp8.fp8_quant_fprop_operands(xt, wt)
    ra = (fp8.fp8_quant_act_1x128_bf16 if xb else fp8.fp8_quant_act_1x128)(xt)
    rb = (fp8.fp8_quant_weight_128x128_bf16 if wb else fp8.fp8_quant_weight_128x128)(wt)
    for got, ref, what in ((qa, ra[0], "qa"), (sa, ra[1], "sa"), (qb, rb[0], "qb"), (sb, rb[1], "sb")):
        g, r = host(got), host(ref)
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8)), what
    # the oracle on the values the kernels saw (bf16 inputs widen exactly)
    xo = xt.float().cpu().numpy()
    wo = wt.float().cpu().numpy()
    if M > 0:
        assert_same(qa, sa, *quant.quant_act_1x128(xo), f"fprop act {M}x{K}")
    if N > 0:
        assert_same(qb, sb, *quant.quant_weight_128x128(wo), f"fprop weight {N}x{K}")


def test_fprop_operands_full_size_dense_fprop():
    x, w = workloads.dense_fprop()
    qa, sa, qb, sb = fp8.fp8_quant_fprop_operands(dev(x), dev(w))
    assert_same(qa, sa, *quant.quant_act_1x128(x), "fprop act full size")
    assert_same(qb, sb, *quant.quant_weight_128x128(w), "fprop weight full size")
