"""Pins of the decode-tiled layout's oracle (oracle/layout.py).

The layout is the library's own storage order (fp8fg.h, fp8_tile_weights_decode);
these tests check what its definition implies, on index-valued inputs so that
every byte's origin can be read back."""
import numpy as np

from oracle import layout


def _index_codes(G, N, K):
    """Every position holds its own flat index, so the output names its source."""
    return np.arange(G * N * K, dtype=np.int64).reshape(G, N, K)


def test_is_a_permutation():
    q = _index_codes(2, 512, 192)
    out = layout.tile_weights_decode(q)
    assert out.shape == (2, 2, 3, 16384)
    assert np.array_equal(np.sort(out.ravel()), np.arange(q.size))


def test_each_block_holds_its_rows_and_k_piece():
    G, N, K = 2, 512, 320
    q = _index_codes(G, N, K)
    out = layout.tile_weights_decode(q)
    for g in range(G):
        for t in range(N // 256):
            for h in range(K // 64):
                src = out[g, t, h]
                e = src - g * N * K
                rows, ks = e // K, e % K
                assert np.array_equal(np.unique(rows), np.arange(256 * t, 256 * t + 256)), (g, t, h)
                assert np.array_equal(np.unique(ks), np.arange(64 * h, 64 * h + 64)), (g, t, h)
                # row r of the n-tile occupies bytes 64 r .. 64 r + 63 of the block
                assert np.array_equal(rows.reshape(256, 64), np.repeat(np.arange(256 * t, 256 * t + 256), 64)
                                      .reshape(256, 64))


def test_chunks_move_whole():
    """Inside a row's 64 bytes only whole 16-byte chunks are reordered: each
    16-byte position holds 16 consecutive K bytes starting on a multiple of 16."""
    G, N, K = 1, 256, 128
    q = _index_codes(G, N, K)
    out = layout.tile_weights_decode(q).reshape(1, 1, 2, 256, 4, 16)
    k = out % K
    assert np.all(np.diff(k, axis=-1) == 1)
    assert np.all(k[..., 0] % 16 == 0)


def test_first_rows_hand_worked():
    """Position s of rows 0-15 holds chunk c (worked by hand from the
    definition: c = s xor ((r >> 2) & 3)): rows 0-3 keep the order, rows 4-7
    swap neighbours, rows 8-11 swap halves, rows 12-15 reverse."""
    expected = {0: [0, 1, 2, 3], 4: [1, 0, 3, 2], 8: [2, 3, 0, 1], 12: [3, 2, 1, 0]}
    q = _index_codes(1, 256, 64)
    out = layout.tile_weights_decode(q).reshape(256, 4, 16)
    for base, order in expected.items():
        for r in range(base, base + 4):
            got = [int(out[r, s, 0] % 64) // 16 for s in range(4)]
            assert got == order, (r, got)
    # the pattern repeats every 16 rows
    assert np.array_equal(out[16:32] % 64, out[0:16] % 64)
