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
                # unit u = 4 w + 2 n + j: 32 rows from 256 t + 64 w + 32 n, 32 K bytes from 64 h + 32 j
                for u in range(16):
                    w, n, j = u // 4, (u // 2) % 2, u % 2
                    ur, uk = rows[1024 * u:1024 * (u + 1)], ks[1024 * u:1024 * (u + 1)]
                    r0, k0 = 256 * t + 64 * w + 32 * n, 64 * h + 32 * j
                    assert np.array_equal(np.unique(ur), np.arange(r0, r0 + 32)), (g, t, h, u)
                    assert np.array_equal(np.unique(uk), np.arange(k0, k0 + 32)), (g, t, h, u)


def test_chunks_move_whole():
    """Only whole 16-byte pieces are moved: each 16-byte position holds 16
    consecutive K bytes of one row, starting on a multiple of 16."""
    G, N, K = 1, 256, 128
    q = _index_codes(G, N, K)
    out = layout.tile_weights_decode(q).reshape(-1, 16)
    assert np.all(np.diff(out, axis=-1) == 1)
    assert np.all((out[:, 0] % K) % 16 == 0)


def test_first_units_hand_worked():
    """Pieces of the first block worked by hand from the definition: (unit,
    piece) -> (row, first K byte).  Pieces 0-31 of a unit walk its 32 rows at
    the unit's first 16 K bytes, pieces 32-63 the same rows 16 bytes on."""
    K = 128
    q = _index_codes(1, 256, K)
    out = layout.tile_weights_decode(q)[0, 0, 0].reshape(16, 64, 16)
    expected = {(0, 0): (0, 0), (0, 1): (1, 0), (0, 31): (31, 0), (0, 32): (0, 16), (0, 63): (31, 16),
                (1, 0): (0, 32), (1, 32): (0, 48), (2, 0): (32, 0), (2, 33): (33, 16), (3, 63): (63, 48),
                (4, 0): (64, 0), (7, 5): (101, 32), (15, 63): (255, 48)}
    for (u, l), (row, k0) in expected.items():
        assert int(out[u, l, 0]) == row * K + k0, (u, l, int(out[u, l, 0]) // K, int(out[u, l, 0]) % K)
    # the second K piece (h = 1) of the same n-tile: the same pieces 64 bytes on
    out1 = layout.tile_weights_decode(q)[0, 0, 1].reshape(16, 64, 16)
    assert np.array_equal(out1 - out, np.full(out.shape, 64))
