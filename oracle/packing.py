"""Packing 2-bit codes four to a byte (oracle; test infrastructure only).

The pages state the storage cost, not a byte layout: the ModelScope card
("Method", recursive residual quantization, and "Model details") gives 2 bits
per real parameter for T = 2, and the zhichai.net note's storage table
("Industry implications") gives 1 bit per real parameter per stage.  An n x m
complex matrix replaces 4nm real parameters, and U and W each hold n*m codes of
2 bits per stage, so T stages cost T*n*m/2 bytes, i.e. T bits per real
parameter.

Layout (a reading; the pages fix none): packed[i][t][M][...] holds the codes of
complex row i, stage t, matrix M (0 = U, 1 = W) as little-endian 32-bit words of
16 codes each.  Word w covers j = 16w .. 16w+15, and code 16w+p sits in bits
8*(p % 4) + 2*(p // 4) .. +1: byte b of the word holds codes b, b+4, b+8, b+12 in
its bit pairs 0-1, 2-3, 4-5, 6-7.  Still four codes per byte and m/4 bytes per
(row, stage, matrix).
"""
from __future__ import annotations

import numpy as np


def packed_nbytes(n: int, m: int, T: int) -> int:
    return T * 2 * n * (m // 4)


def pack(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [T][2][n][m] (values 0..3, m % 16 == 0) -> packed uint8 [n][T][2][m/4]."""
    codes = np.asarray(codes)
    T, two, n, m = codes.shape
    assert two == 2 and m % 16 == 0
    assert int(codes.max(initial=0)) <= 3
    out = np.zeros((n, T, 2, m // 4), dtype=np.uint8)
    for t in range(T):
        for M in range(2):
            # [n][word][p // 4][p % 4]: byte b of a word gathers codes b, b+4, b+8, b+12
            c = codes[t, M].astype(np.uint32).reshape(n, m // 16, 4, 4)
            byte = c[:, :, 0, :] | (c[:, :, 1, :] << 2) | (c[:, :, 2, :] << 4) | (c[:, :, 3, :] << 6)
            out[:, t, M, :] = byte.reshape(n, m // 4).astype(np.uint8)
    return out


def unpack(packed: np.ndarray) -> np.ndarray:
    """packed uint8 [n][T][2][m/4] -> codes uint8 [T][2][n][m]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, T, two, q = packed.shape
    assert two == 2 and q % 4 == 0
    m = 4 * q
    out = np.zeros((T, 2, n, m), dtype=np.uint8)
    for t in range(T):
        for M in range(2):
            words = packed[:, t, M, :].reshape(n, m // 16, 4).astype(np.uint32)   # [n][word][byte]
            for p in range(16):
                out[t, M, :, p::16] = ((words[:, :, p % 4] >> (2 * (p // 4))) & 3).astype(np.uint8)
    return out
