"""Pins for the oracle's fine-grained quantizers (CPU only)."""
import numpy as np

from oracle import e4m3, quant
from tests.goldens import quant_tile_cases
import workloads


def _outlier_acts(rows, K, seed):
    rng = np.random.default_rng(seed)
    return workloads.activations(rng, rows, K, 0.01, 100.0)


def test_golden_tiles():
    for name, tile, scale, codes in quant_tile_cases():
        x = np.tile(tile, (2, 2))                # two rows, two K-blocks each
        q, s = quant.quant_act_1x128(x)
        assert s.shape == (2, 2)
        assert np.all(s.view(np.uint32) == np.float32(scale).view(np.uint32)), name
        for r in range(2):
            for kb in range(2):
                assert np.array_equal(q[r, kb * 128:(kb + 1) * 128], codes), name


def test_float32_division_is_correctly_rounded():
    """The oracle's float32 steps equal float64 division rounded once to float32
    (double rounding is harmless for division from 53 to 24 bits)."""
    x = _outlier_acts(64, 1024, 2)
    q, s = quant.quant_act_1x128(x)
    amax = np.abs(x.reshape(64, 8, 128)).max(axis=2)
    s64 = (amax.astype(np.float64) / 448.0).astype(np.float32)
    assert np.array_equal(s.T, s64)
    y64 = (x.reshape(64, 8, 128).astype(np.float64) / s64[..., None].astype(np.float64)).astype(np.float32)
    assert np.array_equal(q, e4m3.encode(y64).reshape(64, 1024))


def test_error_bound_half_ulp():
    """|dec(q)*s - x| <= (ulp(y)/2 + 2^-24 |y|) * s, with y = x/s."""
    x = _outlier_acts(128, 2048, 3)
    q, s = quant.quant_act_1x128(x)
    sf = np.repeat(s.T, 128, axis=1).astype(np.float64)
    y = x / sf
    err = np.abs(e4m3.decode(q) * sf - x)
    assert np.all(err <= (e4m3.ulp_at(y) / 2 + 2.0 ** -24 * np.abs(y)) * sf * (1 + 2.0 ** -40))


def test_scale_hits_448():
    """Every non-zero tile's max-abs element encodes to +-448 (code 0x7E / 0xFE)."""
    x = _outlier_acts(256, 1024, 4)
    q, s = quant.quant_act_1x128(x)
    t = np.abs(x).reshape(256, 8, 128)
    idx = t.argmax(axis=2)
    qt = q.reshape(256, 8, 128)
    top = np.take_along_axis(qt, idx[..., None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)


def test_idempotent_requantization():
    x = _outlier_acts(128, 1024, 5)
    q, s = quant.quant_act_1x128(x)
    xr = quant.dequant32(q, np.repeat(s.T, 128, axis=1))
    q2, s2 = quant.quant_act_1x128(xr)
    assert np.array_equal(q, q2)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))


def test_power_of_two_equivariance_and_sign():
    x = _outlier_acts(64, 512, 6)
    q, s = quant.quant_act_1x128(x)
    for e in (-5, 3):
        qe, se = quant.quant_act_1x128(x * np.float32(2.0 ** e))
        assert np.array_equal(qe, q)
        assert np.array_equal(se, s * np.float32(2.0 ** e))
    qn, sn = quant.quant_act_1x128(-x)
    assert np.array_equal(qn, q ^ 0x80)
    assert np.array_equal(sn, s)


def test_tile_locality():
    """An outlier planted in one tile changes that tile only (the pages' reason
    for small groups)."""
    x = _outlier_acts(8, 1024, 7)
    q, s = quant.quant_act_1x128(x)
    y = x.copy()
    y[3, 300] = 1e5
    q2, s2 = quant.quant_act_1x128(y)
    diff = np.argwhere(q2 != q)
    assert diff.size and np.all(diff[:, 0] == 3) and np.all(diff[:, 1] // 128 == 2)
    sd = np.argwhere(s2 != s)
    assert sd.tolist() == [[2, 3]]


def test_zero_tile():
    x = np.zeros((2, 256), np.float32)
    x[1, 5] = -0.0
    x[0, 200] = 3.0
    q, s = quant.quant_act_1x128(x)
    assert s[0, 0] == 0 and s[0, 1] == 0
    assert q[1, 5] == 0x80 and np.sum(q[:, :128] & 0x7F) == 0


def test_weight_blocks_match_hand_definition():
    rng = np.random.default_rng(8)
    w = workloads.weights(rng, 256, 384)
    w[130, 7] = 5.0
    q, s = quant.quant_weight_128x128(w)
    assert s.shape == (2, 3)
    for nb in range(2):
        for kb in range(3):
            blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            sv = np.float32(np.abs(blk).max()) / np.float32(448)
            assert s[nb, kb] == sv
            assert np.array_equal(q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128],
                                  e4m3.encode(blk / sv))


def test_weight_transpose_invariance():
    """Square blocks: quantizing W^T gives the transpose of quantizing W."""
    rng = np.random.default_rng(9)
    w = workloads.weights(rng, 384, 256)
    q, s = quant.quant_weight_128x128(w)
    qt, st = quant.quant_weight_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)
    q2, s2 = quant.quant_weight_128x128(w, transpose_out=True)
    assert np.array_equal(q2, q.T) and np.array_equal(s2, s.T)


def test_tokenwise_tiles_run_along_tokens():
    rng = np.random.default_rng(10)
    x = workloads.activations(rng, 256, 64, 0.0, 1.0)
    x[130, 9] = 77.0                                      # token 130 lies in token-tile 1
    q, s = quant.quant_act_1x128_tokenwise(x)
    assert q.shape == (64, 256) and s.shape == (2, 64)
    assert s[1, 9] == np.float32(77.0) / np.float32(448.0)
    assert q[9, 130] == 0x7E
    col = x[0:128, 9]
    assert s[0, 9] == np.float32(np.abs(col).max()) / np.float32(448.0)


def test_fine_grained_beats_per_tensor_on_outliers():
    """An outlier channel large enough to push ordinary values into E4M3's
    subnormal range ruins per-tensor scaling; 1x128 tiles without the outlier
    keep their own scale and their 3-bit relative precision."""
    rng = np.random.default_rng(11)
    K = 2048
    x = rng.standard_normal((256, K), dtype=np.float32)
    x[:, 1000] *= np.float32(1e4)
    normal = np.ones(K, bool)
    normal[1000] = False
    q, s = quant.quant_act_1x128(x)
    rel_fine = np.abs(quant.dequant_act(q, s) - x)[:, normal] / np.abs(x[:, normal])
    qt, st = quant.quant_per_tensor(x)
    rel_coarse = np.abs(e4m3.decode(qt) * np.float64(st) - x)[:, normal] / np.abs(x[:, normal])
    assert np.median(rel_fine) < 2.0 ** -4
    assert rel_coarse.mean() > 4 * rel_fine.mean()


# ---------------------------------------------------------------------------
# Partial groups (axis length not a multiple of 128): the last group is the
# elements that exist; pinned against the exact rational group quantizer.
from tests.bruteforce import quant_group  # noqa: E402


def test_partial_row_groups_brute_force():
    x = _outlier_acts(3, 208, 21)                     # groups of 128 and 80
    x[1, 128:] *= 1e-3
    q, s = quant.quant_act_1x128(x)
    assert q.shape == (3, 208) and s.shape == (2, 3)
    for r in range(3):
        for kb, (lo, hi) in enumerate(((0, 128), (128, 208))):
            bs, bc = quant_group(x[r, lo:hi])
            assert s[kb, r].view(np.uint32) == bs.view(np.uint32), (r, kb)
            assert q[r, lo:hi].tolist() == bc, (r, kb)


def test_partial_token_groups_brute_force():
    x = _outlier_acts(144, 16, 22)                    # token groups of 128 and 16
    q, s = quant.quant_act_1x128_tokenwise(x)
    assert q.shape == (16, 144) and s.shape == (2, 16)
    for k in range(16):
        for tb, (lo, hi) in enumerate(((0, 128), (128, 144))):
            bs, bc = quant_group(x[lo:hi, k])
            assert s[tb, k].view(np.uint32) == bs.view(np.uint32)
            assert q[k, lo:hi].tolist() == bc


def test_partial_weight_blocks_brute_force():
    rng = np.random.default_rng(23)
    w = workloads.weights(rng, 128, 160)              # blocks 128x128 and 128x32
    w[7, 150] = -0.5
    q, s = quant.quant_weight_128x128(w)
    qt, st = quant.quant_weight_128x128(w, transpose_out=True)
    assert s.shape == (1, 2) and np.array_equal(qt, q.T) and np.array_equal(st, s.T)
    for kb, (lo, hi) in enumerate(((0, 128), (128, 160))):
        bs, bc = quant_group(w[:, lo:hi].reshape(-1))
        assert s[0, kb].view(np.uint32) == bs.view(np.uint32)
        assert q[:, lo:hi].reshape(-1).tolist() == bc


def test_per_tensor_scaling_brute_force():
    """The per-tensor baseline is the method's group step with the whole tensor
    as one group: checked against the exact rational quantizer on a small tensor
    with an outlier, negatives and signed zeros, and on an all-zero tensor."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((5, 37)).astype(np.float32)
    x[2, 3] = 90.0
    x[1, :4] = [0.0, -0.0, 1e-9, -3e-7]
    q, s = quant.quant_per_tensor(x)
    s_ref, codes = quant_group(x.ravel())
    assert np.float32(s) == s_ref
    assert np.array_equal(q.ravel(), np.array(codes, dtype=np.uint8))
    z = np.zeros((3, 4), np.float32)
    z[0, 1] = -0.0
    qz, sz = quant.quant_per_tensor(z)
    assert sz == 0.0 and np.array_equal(qz.ravel(), np.array(quant_group(z.ravel())[1], dtype=np.uint8))
