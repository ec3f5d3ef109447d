"""Phase-aware projection, axis-wise scales and recursive residual quantization
(oracle; test infrastructure only).

Sources:
  * zhichai.net reading note, "Step 2: Phase-aware quantization": codebook
    {+1, -1, +i, -i}; b(w) = argmax over s of Re(w conj(s)); separate real and
    imaginary axis scales; dequantized value s_re*b_re + i*s_im*b_im.
  * same note, "Step 3: Recursive residual quantization": W_q is approximated
    by the sum of T terms, and the residual of stage t+1 is the residual of
    stage t minus the dequantized term of stage t.
  * ModelScope card "Fairy2i-W2", "Method": projection to the nearest fourth
    root of unity by angle; axis-wise scaling; each residual term quantized by
    the same phase-aware mechanism; T = 2 for W2.

Readings taken where the pages are silent or open:
  * Code k in {0,1,2,3} stands for s = i**k = (1, i, -1, -i).  Ties in the
    argmax go to the first codeword in that order.
  * Scale granularity: one (s_re, s_im) pair per output row, per stage, per
    matrix (U or W).  s_re is the mean of |Re r| over the entries whose code is
    on the real axis (k in {0, 2}), s_im the mean of |Im r| over the entries
    on the imaginary axis (k in {1, 3}); an empty axis gets scale 0.  For fixed
    codes this mean is the least-squares scale.
  * The sums S_re, S_im are taken in the fixed order defined by
    `ordered_row_sum`, so that a GPU implementation can reproduce the fp64
    scales bit for bit.
  * U and W are quantized independently, each with its own residual chain.
  * Alternative granularity (per_tensor=True): one (s_re, s_im) pair per stage and matrix
    for the whole matrix, the mean over all its entries on that axis.  The sum combines the
    per-row ordered sums in the same fixed order, with rows in place of columns
    (`ordered_row_sum` over the vector of row sums).
"""
from __future__ import annotations

import numpy as np

from .widely_linear import split

# Number of partial sums in the fixed summation order (see ordered_row_sum).
REDUCE_LANES = 256


def project(r_re: np.ndarray, r_im: np.ndarray) -> np.ndarray:
    """Nearest fourth root of unity by angle ("Step 2").

    Re(w conj(s)) for s = 1, i, -1, -i is (a, b, -a, -b) when w = a + ib, so the
    code is the first index of the maximum of that 4-vector.  Returns uint8 codes.
    """
    a = np.asarray(r_re, dtype=np.float64)
    b = np.asarray(r_im, dtype=np.float64)
    scores = np.stack([a, b, -a, -b], axis=0)
    return np.argmax(scores, axis=0).astype(np.uint8)   # argmax returns the first maximum


def ordered_row_sum(v: np.ndarray) -> np.ndarray:
    """Row sums of v ([rows][m], fp64) in the pinned order.

    Lane l in [0, 256) adds v[:, l], v[:, l+256], v[:, l+512], ... one after
    another, starting from +0.0.  Then, for off = 128, 64, ..., 1, lane l < off
    replaces its partial by partial[l] + partial[l+off].  The result is lane 0.
    (Columns beyond m count as +0.0.)
    """
    v = np.asarray(v, dtype=np.float64)
    rows, m = v.shape
    L = REDUCE_LANES
    chunks = max(1, -(-m // L))
    padded = np.zeros((rows, chunks * L), dtype=np.float64)
    padded[:, :m] = v
    p = np.zeros((rows, L), dtype=np.float64)
    for c in range(chunks):
        p = p + padded[:, c * L:(c + 1) * L]
    off = L // 2
    while off >= 1:
        p = p[:, :off] + p[:, off:2 * off]
        off //= 2
    return p[:, 0]


def _tensor_mean(row_sums: np.ndarray, row_counts: np.ndarray) -> float:
    """Per-tensor mean: the row sums combined in the pinned order, over the total count."""
    total = float(ordered_row_sum(np.asarray(row_sums, dtype=np.float64)[None, :])[0])
    count = int(np.sum(row_counts))
    return total / count if count > 0 else 0.0


def _stage(r_re: np.ndarray, r_im: np.ndarray, per_tensor: bool = False):
    """One quantization stage on residual r (rows x m): codes, fp64 scales, new residual."""
    k = project(r_re, r_im)
    on_re = (k == 0) | (k == 2)
    on_im = ~on_re
    n_re = on_re.sum(axis=1)
    n_im = on_im.sum(axis=1)
    s_sum_re = ordered_row_sum(np.where(on_re, np.abs(r_re), 0.0))
    s_sum_im = ordered_row_sum(np.where(on_im, np.abs(r_im), 0.0))
    if per_tensor:
        s_re = np.full(r_re.shape[0], _tensor_mean(s_sum_re, n_re))
        s_im = np.full(r_re.shape[0], _tensor_mean(s_sum_im, n_im))
    else:
        s_re = np.where(n_re > 0, s_sum_re / np.maximum(n_re, 1), 0.0)
        s_im = np.where(n_im > 0, s_sum_im / np.maximum(n_im, 1), 0.0)
    # r <- r - w_hat with w_hat = s_re*b_re + i*s_im*b_im ("Step 3")
    sr = s_re[:, None]
    si = s_im[:, None]
    new_re = np.where(k == 0, r_re - sr, np.where(k == 2, r_re + sr, r_re))
    new_im = np.where(k == 1, r_im - si, np.where(k == 3, r_im + si, r_im))
    return k, s_re, s_im, new_re, new_im


def quantize(R: np.ndarray, T: int, per_tensor: bool = False):
    """Quantize a real weight R [2n][2m] with T residual stages (per_tensor: one scale pair per
    stage and matrix, repeated on every row of the scale arrays).

    Returns (codes, scales32, scales64, residual_norms):
      codes          uint8 [T][2][n][m]   (matrix index 0 = U, 1 = W)
      scales64       fp64  [n][T][2][2]   (last axis: 0 = real-axis scale, 1 = imaginary)
      scales32       fp32, same layout, round-to-nearest-even of scales64
      residual_norms fp64  [2][T+1]       Frobenius norm of the residual before each stage
                                          and after the last one, per matrix
    """
    assert 1 <= T
    U, W = split(R)
    n, m = U.shape
    codes = np.zeros((T, 2, n, m), dtype=np.uint8)
    scales64 = np.zeros((n, T, 2, 2), dtype=np.float64)
    norms = np.zeros((2, T + 1), dtype=np.float64)
    for M, Z in enumerate((U, W)):
        r_re = np.real(Z).copy()
        r_im = np.imag(Z).copy()
        norms[M, 0] = np.sqrt(np.sum(r_re * r_re) + np.sum(r_im * r_im))
        for t in range(T):
            k, s_re, s_im, r_re, r_im = _stage(r_re, r_im, per_tensor)
            codes[t, M] = k
            scales64[:, t, M, 0] = s_re
            scales64[:, t, M, 1] = s_im
            norms[M, t + 1] = np.sqrt(np.sum(r_re * r_re) + np.sum(r_im * r_im))
    return codes, scales64.astype(np.float32), scales64, norms


def dequantize(codes: np.ndarray, scales: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Sum over stages of s_re*b_re + i*s_im*b_im ("Step 2" dequantization, "Step 3" sum).

    codes uint8 [T][2][n][m]; scales [n][T][2][2] (any float type, widened to fp64).
    Returns (U_hat, W_hat), complex128 [n][m].
    """
    T = codes.shape[0]
    s = np.asarray(scales, dtype=np.float64)
    out = []
    for M in range(2):
        acc = np.zeros(codes.shape[2:], dtype=np.complex128)
        for t in range(T):
            k = codes[t, M].astype(np.int64)
            b_re = np.where(k == 0, 1.0, np.where(k == 2, -1.0, 0.0))
            b_im = np.where(k == 1, 1.0, np.where(k == 3, -1.0, 0.0))
            acc = acc + (s[:, t, M, 0][:, None] * b_re + 1j * s[:, t, M, 1][:, None] * b_im)
        out.append(acc)
    return out[0], out[1]


def dequantize_real(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The real form R^ [2n][2m] (fp64) of a quantized layer: the stage sums of "Step 2"
    dequantization ("Step 3": the layer is the sum of its stage terms), mapped back to the real
    blocks by the inverse of the "Step 1" split."""
    from .widely_linear import unsplit
    U, W = dequantize(codes, scales)
    return unsplit(U, W)
