"""Widely-linear GEMV with quantized U, W (oracle; test infrastructure only).

Computes y = sum over t of ( U~(t) x + W~(t) conj(x) ), the inference map of
the pages:
  * ModelScope card "Fairy2i-W2", "Method": y = U x + W conj(x), with each
    matrix replaced by its sum of T quantized residual terms;
  * zhichai.net note, "Step 2" dequantization s_re*b_re + i*s_im*b_im and
    "Industry implications: multiplication-free inference" (B_re, B_im in
    {-1, 0, 1}; a product with +-i is a swap of real and imaginary parts);
  * 36Kr article, the paragraph on parallel stages: the T terms are data
    independent and are simply summed.

Inputs are exactly what the GPU reads: the packed codes' values (as an unpacked
code array), the fp32 scales (widened to fp64 here) and x; x~ = [Re x; Im x]
per batch column, and the result is y~ = [Re y; Im y] per batch column.
"""
from __future__ import annotations

import numpy as np

from .widely_linear import unsplit


def code_planes(k: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Ternary planes of a code array: s = i**k gives b_re = Re s, b_im = Im s in {-1, 0, 1}."""
    k = np.asarray(k).astype(np.int64)
    b_re = np.where(k == 0, 1, np.where(k == 2, -1, 0)).astype(np.int64)
    b_im = np.where(k == 1, 1, np.where(k == 3, -1, 0)).astype(np.int64)
    return b_re, b_im


def _materialize(codes: np.ndarray, scales: np.ndarray, t: int, M: int) -> np.ndarray:
    s = np.asarray(scales, dtype=np.float64)
    b_re, b_im = code_planes(codes[t, M])
    return s[:, t, M, 0][:, None] * b_re + 1j * (s[:, t, M, 1][:, None] * b_im)


def gemv_ref(codes: np.ndarray, scales: np.ndarray, x: np.ndarray, stages=None) -> np.ndarray:
    """y~ [B][2n] (fp64) for codes uint8 [T][2][n][m], scales [n][T][2][2], x [B][2m].

    `stages` optionally restricts the sum to a subset of stage indices.
    """
    T, _, n, m = codes.shape
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    assert x.shape[1] == 2 * m
    xc = x[:, :m] + 1j * x[:, m:]              # [B][m]
    y = np.zeros((x.shape[0], n), dtype=np.complex128)
    for t in (range(T) if stages is None else stages):
        Ut = _materialize(codes, scales, t, 0)
        Wt = _materialize(codes, scales, t, 1)
        y = y + xc @ Ut.T + np.conj(xc) @ Wt.T
    return np.concatenate([y.real, y.imag], axis=1)


def gemv_ref_real(codes: np.ndarray, scales: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Second route: rebuild the real matrix R^ of the quantized layer and apply it to x~."""
    T = codes.shape[0]
    U = sum(_materialize(codes, scales, t, 0) for t in range(T))
    W = sum(_materialize(codes, scales, t, 1) for t in range(T))
    Rhat = unsplit(U, W)
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    return x @ Rhat.T
