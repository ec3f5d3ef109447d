"""Real <-> widely-linear complex reparameterization (oracle; test infrastructure only).

Follows the zhichai.net reading note, "Step 1: Widely-linear transformation",
Theorem 1: a real map y~ = R x~ with R of size 2n x 2m equals the complex map
y = U x + W conj(x), and the note prints U, W as half-sums of R's four blocks.
The ModelScope card ("Method", widely-linear transform) states the same map and
calls it lossless and unique.

Reading taken where the pages are silent: R11, R12, R21, R22 are the four
quadrants of R (R11 = R[:n, :m], R12 = R[:n, m:], R21 = R[n:, :m],
R22 = R[n:, m:]), so that x~ = [Re x; Im x] and y~ = [Re y; Im y].
"""
from __future__ import annotations

import numpy as np


def split(R: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """R (real, [2n][2m]) -> (U, W), complex128 [n][m].

    Closed form of Theorem 1 ("Step 1"), each block entry widened exactly to fp64:
        Re U = (R11 + R22)/2     Im U = (R21 - R12)/2
        Re W = (R11 - R22)/2     Im W = (R12 + R21)/2
    The sum is formed first and then halved (multiplication by 0.5), in that order.
    """
    R = np.asarray(R)
    two_n, two_m = R.shape
    assert two_n % 2 == 0 and two_m % 2 == 0, "R must have even dimensions"
    n, m = two_n // 2, two_m // 2
    R = R.astype(np.float64)
    A, B = R[:n, :m], R[:n, m:]     # R11, R12
    C, D = R[n:, :m], R[n:, m:]     # R21, R22
    U = ((A + D) * 0.5) + 1j * ((C - B) * 0.5)
    W = ((A - D) * 0.5) + 1j * ((B + C) * 0.5)
    return U, W


def unsplit(U: np.ndarray, W: np.ndarray) -> np.ndarray:
    """(U, W) -> R, the inverse of `split`.

    Not printed on the pages; it follows from expanding U x + W conj(x) with
    x = a + ib into real and imaginary parts (the equivalence of "Step 1"):
        R11 = Re U + Re W    R12 = Im W - Im U
        R21 = Im U + Im W    R22 = Re U - Re W
    """
    Ur, Ui = np.real(U).astype(np.float64), np.imag(U).astype(np.float64)
    Wr, Wi = np.real(W).astype(np.float64), np.imag(W).astype(np.float64)
    top = np.concatenate([Ur + Wr, Wi - Ui], axis=1)
    bot = np.concatenate([Ui + Wi, Ur - Wr], axis=1)
    return np.concatenate([top, bot], axis=0)
