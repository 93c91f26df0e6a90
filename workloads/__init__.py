"""Seeded synthetic inputs for the five workloads (shared by tests, smoke and bench).

This module only draws random numbers and shapes; it holds none of the
quantization or GEMM arithmetic, so both the CPU oracle and the HIP path can
take their inputs from it.

Recipes (sigma is a standard deviation):
  dense_small   M=128  N=256  K=512   A ~ N(0,1), 0.5% of channels x50; W ~ N(0,0.02)
  dense_fprop   M=4096 N=7168 K=2048  A ~ N(0,1), 0.1% of channels x100; W ~ N(0,0.02)
  linear_trio   7168->2048 linear at 8192 tokens: X ~ N(0,1) (0.1% channels x100),
                W ~ N(0,0.02) [2048][7168], dY ~ N(0,1e-3) [8192][2048]
  moe_contig    32 experts, 8192 tokens x top-8 = 65536 routed rows, counts
                multinomial with Zipf(1.1) weights over a seeded expert ranking,
                each group padded to a multiple of 128 rows (pad rows zero);
                gate+up K=7168 N=4096; expert weights ~ N(0,0.02)
  moe_masked    32 experts, 128-row padded buffers, valid rows U{1..64};
                gate+up K=7168 N=4096 and down K=2048 N=7168; rows past the
                valid count hold garbage
Outlier channels: max(1, round(frac * K)) distinct channel indices drawn
without replacement; the whole column is multiplied by the factor.
"""

import numpy as np

SEEDS = {"dense_small": 101, "dense_fprop": 102, "linear_trio": 103,
         "moe_contig": 104, "moe_masked": 105, "moe_gate_up": 106, "moe_down": 107}

SHAPES = {
    "dense_small": dict(M=128, N=256, K=512, outlier_frac=0.005, outlier_mult=50.0),
    "dense_fprop": dict(M=4096, N=7168, K=2048, outlier_frac=0.001, outlier_mult=100.0),
    "linear_trio": dict(T=8192, IN=7168, OUT=2048, outlier_frac=0.001, outlier_mult=100.0,
                        dy_sigma=1e-3),
    "moe_contig": dict(G=32, tokens=8192, topk=8, N=4096, K=7168, zipf=1.1,
                       outlier_frac=0.001, outlier_mult=100.0),
    "moe_masked": dict(G=32, M_max=128, lo=1, hi=64, gate_up=(4096, 7168), down=(7168, 2048),
                       outlier_frac=0.001, outlier_mult=100.0),
}


def rngs(seed, n):
    """n independent generators spawned from one seed."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def activations(rng, rows, K, outlier_frac=0.0, outlier_mult=1.0, sigma=1.0):
    """float32 [rows][K] ~ N(0, sigma) with whole outlier channels scaled."""
    x = rng.standard_normal((rows, K), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if outlier_frac > 0:
        n = max(1, int(round(outlier_frac * K)))
        idx = rng.choice(K, size=n, replace=False)
        x[:, idx] *= np.float32(outlier_mult)
    return x


def weights(rng, N, K, sigma=0.02):
    """float32 [N][K] ~ N(0, sigma)."""
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def zipf_counts(rng, rows, G, alpha):
    """Rows per expert: multinomial over G experts with p ~ rank^-alpha, ranks shuffled."""
    ranks = rng.permutation(G) + 1
    p = ranks.astype(np.float64) ** -alpha
    p /= p.sum()
    return rng.multinomial(rows, p).astype(np.int64)


def pad_offsets(counts, align=128):
    """Group offsets (length G+1) after padding every group to a multiple of `align`."""
    padded = (np.asarray(counts, dtype=np.int64) + align - 1) // align * align
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)


def masked_counts(rng, G, lo, hi):
    """Valid rows per expert, uniform on {lo..hi}."""
    return rng.integers(lo, hi + 1, size=G).astype(np.int64)


def dense_small():
    c = SHAPES["dense_small"]
    ra, rb = rngs(SEEDS["dense_small"], 2)
    return (activations(ra, c["M"], c["K"], c["outlier_frac"], c["outlier_mult"]),
            weights(rb, c["N"], c["K"]))


def dense_fprop(seed_offset=0):
    """Activations [4096][2048] and weights [7168][2048]; `seed_offset` gives
    further independent input sets of the same recipe."""
    c = SHAPES["dense_fprop"]
    ra, rb = rngs(SEEDS["dense_fprop"] + 1000 * seed_offset, 2)
    return (activations(ra, c["M"], c["K"], c["outlier_frac"], c["outlier_mult"]),
            weights(rb, c["N"], c["K"]))


def linear_trio():
    """X [8192][7168], W [2048][7168], dY [8192][2048]."""
    c = SHAPES["linear_trio"]
    rx, rw, rd = rngs(SEEDS["linear_trio"], 3)
    x = activations(rx, c["T"], c["IN"], c["outlier_frac"], c["outlier_mult"])
    w = weights(rw, c["OUT"], c["IN"])
    dy = activations(rd, c["T"], c["OUT"], sigma=c["dy_sigma"])
    return x, w, dy


def moe_contig_layout():
    """Per-expert valid counts and padded group offsets for the contiguous layout."""
    c = SHAPES["moe_contig"]
    (rc,) = rngs(SEEDS["moe_contig"], 1)
    counts = zipf_counts(rc, c["tokens"] * c["topk"], c["G"], c["zipf"])
    return counts, pad_offsets(counts)


def moe_contig_rows(counts, offsets, K, seed_stream=1):
    """A rows [M_total][K]: valid rows ~ N(0,1) with outlier channels, padding rows zero."""
    c = SHAPES["moe_contig"]
    (ra,) = rngs(SEEDS["moe_contig"] + seed_stream, 1)
    a = np.zeros((int(offsets[-1]), K), dtype=np.float32)
    x = activations(ra, int(np.sum(counts)), K, c["outlier_frac"], c["outlier_mult"])
    pos = 0
    for g, n in enumerate(counts):
        a[offsets[g]:offsets[g] + n] = x[pos:pos + n]
        pos += n
    return a


def expert_weight(kind, g, N, K):
    """Weights [N][K] of expert g, ~ N(0,0.02), drawn per expert.  `kind` names
    the layer: 'moe_gate_up' (N=4096, K=7168) and 'moe_down' (N=7168, K=2048)
    are shared by the contiguous and masked workloads; any other SEEDS key
    gives an independent set."""
    (rw,) = rngs(SEEDS[kind] * 1000 + 7 + g, 1)
    return weights(rw, N, K)


def moe_masked_inputs(N, K, G=32, M_max=128):
    """(masked_m [G], A [G][M_max][K]); rows >= masked_m[g] hold garbage."""
    c = SHAPES["moe_masked"]
    rc, ra = rngs(SEEDS["moe_masked"] + K, 2)
    m = masked_counts(rc, G, c["lo"], c["hi"])
    a = np.empty((G, M_max, K), dtype=np.float32)
    for g in range(G):
        a[g] = activations(ra, M_max, K, c["outlier_frac"], c["outlier_mult"])
        a[g, m[g]:] = rng_garbage(ra, M_max - int(m[g]), K)
    return m, a


def rng_garbage(rng, rows, K):
    """Large-magnitude noise for rows that must never be read."""
    return (rng.standard_normal((rows, K), dtype=np.float32) * np.float32(1e4))
