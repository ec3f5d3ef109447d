"""Prefill path: per-token int8 activations and the ternary-plane integer GEMM
(oracle; test infrastructure only).

The pages give the arithmetic only as "B_re, B_im in {-1, 0, 1}; the matrix
product becomes additions, subtractions and skips" (zhichai.net note,
"Industry implications: multiplication-free inference").  The int8 activation
format is not on the pages; it is the plainest reading of a batched prefill
product on integer matrix units:

  * per token: amax = max |x~_j| over all 2m reals, delta = fl32(amax / 127),
    q_j = clamp(round_half_even(fl32(x~_j / delta)), -127, 127); a token with
    delta == 0 gets q = 0.
  * P[t][M][plane][comp][tok][i] = sum_j B_plane(t, M)[i, j] * q_comp[tok][j],
    plane 0 = B_re, 1 = B_im; comp 0 = the first m reals of x~ (a = Re x),
    comp 1 = the last m (b = Im x).
  * y~ = delta * (the widely-linear combination of P with the fp32 scales),
    which is the GEMV of gemv.py applied to x = delta * q.
"""
from __future__ import annotations

import numpy as np

from .gemv import code_planes


def act_quant_ref(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x [N][2m] (exact values of bf16 / fp32 inputs) -> (q int8 [N][2m], delta fp32 [N]).

    fp32 divisions are emulated as an fp64 division rounded once to fp32; with
    53 >= 2*24 + 2 mantissa bits this equals the correctly rounded fp32 result.
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=1)
    delta = (amax / 127.0).astype(np.float32)
    q = np.zeros(x.shape, dtype=np.int8)
    for tok in range(x.shape[0]):
        d = float(delta[tok])
        if d == 0.0:
            continue
        ratio = (x[tok] / d).astype(np.float32).astype(np.float64)
        q[tok] = np.clip(np.rint(ratio), -127, 127).astype(np.int8)   # rint: ties to even
    return q, delta


def gemm_int_ref(codes: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Raw accumulators int64 [T][2][2][2][N][n] via fp64 matrix products.

    Every partial sum is an integer of magnitude <= 127*m < 2**53, so the fp64
    products are exact.
    """
    T, _, n, m = codes.shape
    q = np.asarray(q).astype(np.float64)
    comps = (q[:, :m], q[:, m:])                 # [N][m] each
    N = q.shape[0]
    out = np.zeros((T, 2, 2, 2, N, n), dtype=np.int64)
    for t in range(T):
        for M in range(2):
            planes = code_planes(codes[t, M])
            for p in range(2):
                Bp = planes[p].astype(np.float64)      # [n][m]
                for c in range(2):
                    out[t, M, p, c] = np.rint(comps[c] @ Bp.T).astype(np.int64)
    return out


def gemm_int_ref_loops(codes: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Same result as gemm_int_ref with explicit int64 loops (tiny shapes only)."""
    T, _, n, m = codes.shape
    N = q.shape[0]
    q = np.asarray(q).astype(np.int64)
    out = np.zeros((T, 2, 2, 2, N, n), dtype=np.int64)
    for t in range(T):
        for M in range(2):
            b_re, b_im = code_planes(codes[t, M])
            for p, Bp in enumerate((b_re, b_im)):
                for c in range(2):
                    for tok in range(N):
                        for i in range(n):
                            acc = 0
                            for j in range(m):
                                acc += int(Bp[i, j]) * int(q[tok, c * m + j])
                            out[t, M, p, c, tok, i] = acc
    return out


def gemm_epilogue_ref(P: np.ndarray, scales: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """y~ [N][2n] fp64 from raw accumulators P [T][2][2][2][N][n], fp32 scales and delta.

    With x = a + ib and quantized terms s_re*b_re + i*s_im*b_im:
      U x       : Re = sUr*P(U,re,a) - sUi*P(U,im,b)   Im = sUi*P(U,im,a) + sUr*P(U,re,b)
      W conj(x) : Re = sWr*P(W,re,a) + sWi*P(W,im,b)   Im = sWi*P(W,im,a) - sWr*P(W,re,b)
    summed over stages and multiplied by the token's delta.
    """
    P = np.asarray(P).astype(np.float64)
    s = np.asarray(scales, dtype=np.float64)
    T = P.shape[0]
    N, n = P.shape[4], P.shape[5]
    y_re = np.zeros((N, n))
    y_im = np.zeros((N, n))
    for t in range(T):
        sUr, sUi = s[:, t, 0, 0], s[:, t, 0, 1]
        sWr, sWi = s[:, t, 1, 0], s[:, t, 1, 1]
        y_re += sUr * P[t, 0, 0, 0] - sUi * P[t, 0, 1, 1] + sWr * P[t, 1, 0, 0] + sWi * P[t, 1, 1, 1]
        y_im += sUi * P[t, 0, 1, 0] + sUr * P[t, 0, 0, 1] + sWi * P[t, 1, 1, 0] - sWr * P[t, 1, 0, 1]
    d = np.asarray(delta, dtype=np.float64)[:, None]
    return np.concatenate([d * y_re, d * y_im], axis=1)
