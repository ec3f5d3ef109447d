"""Packing 2-bit codes four to a byte (oracle; test infrastructure only).

The pages state the storage cost, not a byte layout: the ModelScope card
("Method", recursive residual quantization, and "Model details") gives 2 bits
per real parameter for T = 2, and the zhichai.net note's storage table
("Industry implications") gives 1 bit per real parameter per stage.  An n x m
complex matrix replaces 4nm real parameters, and U and W each hold n*m codes of
2 bits per stage, so T stages cost T*n*m/2 bytes, i.e. T bits per real
parameter.

Layout (a reading; the pages fix none): packed[i][t][M][q], byte q of complex
row i, stage t, matrix M (0 = U, 1 = W), holds codes j = 4q .. 4q+3 with code
4q+r in bits 2r, 2r+1 (least significant first).
"""
from __future__ import annotations

import numpy as np


def packed_nbytes(n: int, m: int, T: int) -> int:
    return T * 2 * n * (m // 4)


def pack(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [T][2][n][m] (values 0..3, m % 4 == 0) -> packed uint8 [n][T][2][m/4]."""
    codes = np.asarray(codes)
    T, two, n, m = codes.shape
    assert two == 2 and m % 4 == 0
    assert int(codes.max(initial=0)) <= 3
    out = np.zeros((n, T, 2, m // 4), dtype=np.uint8)
    for t in range(T):
        for M in range(2):
            c = codes[t, M].astype(np.uint32).reshape(n, m // 4, 4)
            byte = c[:, :, 0] | (c[:, :, 1] << 2) | (c[:, :, 2] << 4) | (c[:, :, 3] << 6)
            out[:, t, M, :] = byte.astype(np.uint8)
    return out


def unpack(packed: np.ndarray) -> np.ndarray:
    """packed uint8 [n][T][2][m/4] -> codes uint8 [T][2][n][m]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, T, two, q = packed.shape
    assert two == 2
    out = np.zeros((T, 2, n, 4 * q), dtype=np.uint8)
    for t in range(T):
        for M in range(2):
            b = packed[:, t, M, :].astype(np.uint32)
            for r in range(4):
                out[t, M, :, r::4] = ((b >> (2 * r)) & 3).astype(np.uint8)
    return out
