"""Packing 2-bit codes four to a byte (oracle; test infrastructure only).

The pages state the storage cost, not a byte layout: the ModelScope card
("Method", recursive residual quantization, and "Model details") gives 2 bits
per real parameter for T = 2, and the zhichai.net note's storage table
("Industry implications") gives 1 bit per real parameter per stage.  An n x m
complex matrix replaces 4nm real parameters, and U and W each hold n*m codes of
2 bits per stage, so T stages cost T*n*m/2 bytes, i.e. T bits per real
parameter.

Layout (a reading; the pages fix none), in two levels.

Words.  The codes of complex row i, stage t, matrix M (0 = U, 1 = W) are cut into
little-endian 32-bit words of 16 consecutive codes: word w covers columns
j = 16w .. 16w+15, and code 16w+p sits in bits 8*(p % 4) + 2*(p // 4) .. +1, so
byte b of the word holds codes b, b+4, b+8, b+12 in its bit pairs 0-1, 2-3, 4-5, 6-7.

Word order.  Rows are grouped in tiles of 16 (the last tile padded with rows of
code 0), columns in chunks of 256 (the last chunk may hold 64, 128 or 192) and each
chunk in groups of 64 columns (4 words).  With plane P = 2t + M and G_c the number
of 64-column groups in chunk c, the tile's bytes are ordered

    [chunk c][plane P][group g < G_c][row r < 16][word w < 4]

so one (tile, chunk, plane) block is 16 rows x G_c groups of 16 bytes.  Tiles follow
one another.  Four codes per byte still, m/4 bytes per (row, plane); only the
padding rows of the last tile add bytes.
"""
from __future__ import annotations

import numpy as np

TILE_ROWS = 16
CHUNK_COLS = 256
GROUP_COLS = 64


def _tiles(n: int) -> int:
    return -(-n // TILE_ROWS)


def packed_nbytes(n: int, m: int, T: int) -> int:
    """Bytes of the packed form: 16-row tiles, T * 2 planes, m/4 bytes per row and plane."""
    return _tiles(n) * TILE_ROWS * T * 2 * (m // 4)


def pack_words(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [T][2][n][m] (values 0..3, m % 16 == 0) -> words uint32 [T][2][n][m/16]."""
    codes = np.asarray(codes)
    T, two, n, m = codes.shape
    assert two == 2 and m % 16 == 0
    assert int(codes.max(initial=0)) <= 3
    c = codes.astype(np.uint32).reshape(T, 2, n, m // 16, 4, 4)     # [..][word][p // 4][p % 4]
    byte = c[..., 0, :] | (c[..., 1, :] << 2) | (c[..., 2, :] << 4) | (c[..., 3, :] << 6)  # [..][word][b]
    return byte[..., 0] | (byte[..., 1] << 8) | (byte[..., 2] << 16) | (byte[..., 3] << 24)


def _blocks(n: int, m: int, T: int):
    """The layout's blocks in storage order: (tile, plane t, M, first word, words per row)."""
    for tile in range(_tiles(n)):
        for c in range(-(-m // CHUNK_COLS)):
            groups = min(CHUNK_COLS, m - CHUNK_COLS * c) // GROUP_COLS
            for P in range(2 * T):
                for g in range(groups):
                    yield tile, P // 2, P % 2, (CHUNK_COLS * c + GROUP_COLS * g) // 16


def pack(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [T][2][n][m] (m % 64 == 0) -> packed uint8 [packed_nbytes(n, m, T)]."""
    codes = np.asarray(codes)
    T, _, n, m = codes.shape
    assert m % GROUP_COLS == 0
    words = np.zeros((T, 2, _tiles(n) * TILE_ROWS, m // 16), dtype=np.uint32)
    words[:, :, :n] = pack_words(codes)
    pieces = [words[t, M, TILE_ROWS * tile:TILE_ROWS * (tile + 1), w0:w0 + 4]   # [row][word]
              for tile, t, M, w0 in _blocks(n, m, T)]
    out = np.concatenate([p.reshape(-1) for p in pieces]).astype("<u4").view(np.uint8)
    assert out.size == packed_nbytes(n, m, T)
    return out


def unpack(packed: np.ndarray, n: int, m: int, T: int) -> np.ndarray:
    """packed uint8 [packed_nbytes(n, m, T)] -> codes uint8 [T][2][n][m]."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    assert packed.size == packed_nbytes(n, m, T)
    stream = packed.view("<u4")
    words = np.zeros((T, 2, _tiles(n) * TILE_ROWS, m // 16), dtype=np.uint32)
    pos = 0
    for tile, t, M, w0 in _blocks(n, m, T):
        words[t, M, TILE_ROWS * tile:TILE_ROWS * (tile + 1), w0:w0 + 4] = \
            stream[pos:pos + 4 * TILE_ROWS].reshape(TILE_ROWS, 4)
        pos += 4 * TILE_ROWS
    words = words[:, :, :n]
    out = np.zeros((T, 2, n, m), dtype=np.uint8)
    for p in range(16):
        out[..., p::16] = ((words >> (8 * (p % 4) + 2 * (p // 4))) & 3).astype(np.uint8)
    return out
