"""Decode-tiled weight layout (test infrastructure only).

This storage order is the library's own, not the pages'.  The pages define the
masked MoE layout's operation (DeepGEMM launch article, section "Principais
caracteristicas"), and the GEMM on tiled weights must give the same result as
the GEMM on the plain [G][N][K] codes.  The layout only decides where each
byte lies, so that a decode kernel's every step reads one contiguous block.

Definition (the one fp8fg.h states for fp8_tile_weights_decode): for expert g,
n-tile t (rows 256 t .. 256 t + 255) and K piece h (bytes 64 h .. 64 h + 63),
one 16384-byte block, made of sixteen 1024-byte units u = 4 w + 2 n + j
(w = 0..3, n = 0..1, j = 0..1); unit u holds rows 256 t + 64 w + 32 n + i
(i = 0..31) and K bytes 64 h + 32 j .. 64 h + 32 j + 31, as 64 pieces of 16
bytes: piece l (bytes 16 l .. 16 l + 15 of the unit) is row i = l mod 32,
K bytes 64 h + 32 j + 16 (l div 32) .. + 15.  (These are the 16-byte
fragments that lane l of wave w of the decode kernel loads for its MFMA tile
n and K step j, in load order.)

What pins it: the order of the units and pieces is a choice of this library
that the pages cannot fix (parity unpinned against the pages for that
detail).  The tests check the rest against the definition's consequences --
a permutation of the input, each block holding exactly its rows and K piece,
each unit its 32 rows and 32 K bytes, 16-byte pieces moved whole -- and a
hand-worked table of the first units.  On the GPU, the GEMM on tiled weights
must match the GEMM on plain weights bit for bit, and the oracle GEMM's
bound.
"""

import numpy as np

ROWS = 256     # rows of an n-tile
PIECE = 64     # K bytes per block
CHUNK = 16     # bytes moved as one unit


def tile_weights_decode(q):
    """q [G][N][K] (any dtype; codes are u8) -> [G][N/256][K/64][256 * 64],
    the decode-tiled layout."""
    G, N, K = q.shape
    assert N % ROWS == 0 and K % PIECE == 0, "N % 256 == 0 and K % 64 == 0"
    T, H = N // ROWS, K // PIECE
    # row 256 t + 64 w + 32 n + i, K byte 64 h + 32 j + 16 d + b:
    # axes [g][t][w][n][i][h][j][d][b]
    x = q.reshape(G, T, 4, 2, 32, H, 2, 2, CHUNK)
    # block (g, t, h), unit (w, n, j), piece l = 32 d + i, byte b
    x = x.transpose(0, 1, 5, 2, 3, 6, 7, 4, 8)
    return np.ascontiguousarray(x).reshape(G, T, H, ROWS * PIECE)
