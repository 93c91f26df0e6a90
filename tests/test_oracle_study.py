"""Pins for the E5M2 codec and the format / granularity study (CPU only)."""
import numpy as np
import torch

from oracle import e4m3, e5m2, study
import workloads


def test_e5m2_decode_matches_torch_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    ours = e5m2.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], ref[fin])
    assert e5m2.decode(np.uint8(0x7B)) == 57344.0
    assert e5m2.decode(np.uint8(0x01)) == 2.0 ** -16
    assert e5m2.decode(np.uint8(0x04)) == 2.0 ** -14
    assert np.isinf(e5m2.decode(np.uint8(0x7C)))
    assert e5m2.MAGNITUDES.size == 124 and np.all(np.diff(e5m2.MAGNITUDES) > 0)


def test_e5m2_encode_matches_torch_round_to_nearest_even():
    """Below the overflow threshold torch's cast is RNE: compare on random
    values of every binade, on every midpoint and on its float32 neighbours."""
    rng = np.random.default_rng(5)
    parts = []
    for e in range(-20, 16):
        m = rng.integers(0, 1 << 23, size=20000, dtype=np.uint32)
        parts.append(((np.uint32(e + 127) << 23) | m).view(np.float32))
    mids = e5m2.MIDPOINTS.astype(np.float32)
    parts += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))]
    v = np.concatenate(parts)
    v = v[v < 57344.0 + 4096.0]
    v = np.concatenate([v, -v, [0.0, -0.0]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(e5m2.encode(v), ref)
    assert e5m2.encode(np.float32(1e6)) == 0x7B and e5m2.encode(np.float32(-1e6)) == 0xFB


def _on_grid(rng, rows, cols):
    """E4M3 values with a 448 in every 1x128 group along either axis and in every
    128x128 block, so that every E4M3 scheme of the study reproduces it exactly."""
    c = rng.integers(0, 0x7F, size=(rows, cols), dtype=np.uint8) | (rng.integers(0, 2, size=(rows, cols),
                                                                                   dtype=np.uint8) << 7)
    x = e4m3.decode(c).astype(np.float32)
    r = np.arange(rows)[:, None]
    k = np.arange(cols)[None, :]
    x[(r % 128) == (k % 128)] = 448.0
    return x


def test_study_plumbing_is_exact_on_grid_inputs():
    rng = np.random.default_rng(9)
    x, w, dy = _on_grid(rng, 256, 384), _on_grid(rng, 256, 384), _on_grid(rng, 256, 256)
    res = study.run(x, w, dy, schemes=("fine_e4m3", "tensor_e4m3", "fine_hybrid"))
    for g in study.GEMMS:
        assert res["fine_e4m3"][g] == 0.0 and res["tensor_e4m3"][g] == 0.0, g
    assert res["fine_hybrid"]["fprop"] == 0.0          # the hybrid changes only dY
    assert res["fine_hybrid"]["dgrad"] > 0.0 and res["fine_hybrid"]["wgrad"] > 0.0


def test_unified_e4m3_and_fine_groups_win_on_the_linear_layer():
    """The pages' claims, on the first 256 tokens of the linear-layer workload:
    with fine-grained groups E4M3 gradients beat E5M2 ones, and fine groups beat
    one scale per tensor on activations with outlier channels."""
    x, w, dy = workloads.linear_trio()
    res = study.run(x[:256], w, dy[:256])
    for g in ("dgrad", "wgrad"):
        assert res["fine_hybrid"][g] > 1.3 * res["fine_e4m3"][g], (g, res)
        assert res["tensor_hybrid"][g] > 1.3 * res["tensor_e4m3"][g], (g, res)
    assert res["fine_hybrid"]["fprop"] == res["fine_e4m3"]["fprop"]
    assert res["tensor_e4m3"]["fprop"] > 1.2 * res["fine_e4m3"]["fprop"], res


def _exact(vals, mags):
    from tests.bruteforce import quant_dequant_group
    return np.array([float(v) for v in quant_dequant_group(vals, mags)], dtype=np.float64)


def test_e5m2_groups_and_per_tensor_against_exact_quantizer():
    """The study's E5M2 1x128 groups (scale amax / 57344) and its per-tensor
    quantizers (E4M3 and E5M2) equal an exact rational re-implementation: one
    scale per 128 consecutive values (or per tensor), RN32 division, nearest
    format value with ties to even."""
    from tests.bruteforce import MAGS, MAGS_E5M2
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((3, 256)) * np.exp2(rng.integers(-12, 6, size=(3, 256)))).astype(np.float32)
    x[1, 130] = 700.0                       # an outlier in one group only
    x[2, 128:256] = 0.0                     # an all-zero group
    got = study._groups_e5m2(x)
    ref = np.concatenate([_exact(x[r, 128 * j:128 * j + 128], MAGS_E5M2) for r in range(3) for j in range(2)])
    assert np.array_equal(got.ravel(), ref)
    t = x[:2, :64].copy()
    # values 2^20 .. 2^28 below the max-abs: normal in E5M2 only when the
    # scale maps the max-abs to 57344, subnormal or zero with a smaller target
    t[0, :5] = np.max(np.abs(t)) * np.exp2(-np.array([20.0, 22.0, 24.0, 26.0, 28.0])).astype(np.float32)
    assert np.array_equal(study._tensor(t, e5m2).ravel(), _exact(t.ravel(), MAGS_E5M2))
    assert np.array_equal(study._tensor(t, e4m3).ravel(), _exact(t.ravel(), MAGS))
