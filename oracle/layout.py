"""Decode-tiled weight layout (test infrastructure only).

This storage order is the library's own, not the pages'.  The pages define the
masked MoE layout's operation (DeepGEMM launch article, section "Principais
caracteristicas"), and the GEMM on tiled weights must give the same result as
the GEMM on the plain [G][N][K] codes.  The layout only decides where each
byte lies, so that a decode kernel's every step reads one contiguous block.

Definition (the one fp8fg.h states for fp8_tile_weights_decode): for expert g,
n-tile t (rows 256 t .. 256 t + 255) and K piece h (bytes 64 h .. 64 h + 63),
one 16384-byte block; in it, row r of the n-tile takes bytes 64 r .. 64 r + 63,
and the 16-byte position s of that row holds chunk c = s ^ ((r >> 2) & 3) of
the row's 64-byte piece.

What pins it: the chunk order inside a row piece is a choice of this library
that the pages cannot fix (parity unpinned against the pages for that
detail).  The tests check the rest against the definition's consequences --
a permutation of the input, each block holding exactly its rows and K piece,
chunks moved whole -- and a hand-worked table of the first 16 rows.  On the
GPU, the GEMM on tiled weights must match the GEMM on plain weights bit for
bit, and the oracle GEMM's bound.
"""

import numpy as np

ROWS = 256     # rows of an n-tile
PIECE = 64     # K bytes per block
CHUNK = 16     # bytes moved as one unit


def chunk_of(r, s):
    """The chunk of row r's 64-byte piece stored at 16-byte position s."""
    return s ^ ((r >> 2) & 3)


def tile_weights_decode(q):
    """q [G][N][K] (any dtype; codes are u8) -> [G][N/256][K/64][256 * 64],
    the decode-tiled layout."""
    G, N, K = q.shape
    assert N % ROWS == 0 and K % PIECE == 0, "N % 256 == 0 and K % 64 == 0"
    T, H = N // ROWS, K // PIECE
    # [g][t][r][h][s][16]: row r of n-tile t, K piece h, chunk s of the piece
    x = q.reshape(G, T, ROWS, H, PIECE // CHUNK, CHUNK)
    x = x.transpose(0, 1, 3, 2, 4, 5)          # [g][t][h][r][chunk][16]
    r = np.arange(ROWS).reshape(ROWS, 1)
    s = np.arange(PIECE // CHUNK).reshape(1, PIECE // CHUNK)
    src = chunk_of(r, s)                       # [r][s] -> chunk read for position s
    out = np.take_along_axis(x, src.reshape(1, 1, 1, ROWS, PIECE // CHUNK, 1), axis=4)
    return np.ascontiguousarray(out).reshape(G, T, H, ROWS * PIECE)
