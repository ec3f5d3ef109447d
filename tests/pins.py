"""Checks that pin the oracle to facts outside itself.

Each check takes the oracle function(s) it exercises as arguments, so the same
check runs against the real oracle (must pass) and against copies with a
planted mistake (must fail; see test_oracle_mutants.py).  None of them retypes
the oracle's own formula: they use closed forms from the pages, brute force
with Python complex arithmetic, exact identities of the mathematics, or the
hand-worked fixtures under tests/golden/.
"""
from __future__ import annotations

import cmath
import itertools
import math

import numpy as np

import golden_io

CODEWORDS = (1 + 0j, 1j, -1 + 0j, -1j)      # s = i**k


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- split ----

def check_split_identity(split, seed=0, shape=(24, 40), batch=3):
    """U x + W conj(x) == R [Re x; Im x] (Theorem 1), to 1e-12 relative."""
    rng = np.random.default_rng(seed)
    R = rng.standard_normal(shape).astype(np.float32)
    n, m = shape[0] // 2, shape[1] // 2
    U, W = split(R)
    assert U.shape == (n, m) and W.shape == (n, m)
    xt = rng.standard_normal((batch, 2 * m))
    x = xt[:, :m] + 1j * xt[:, m:]
    y = x @ U.T + np.conj(x) @ W.T
    lhs = np.concatenate([y.real, y.imag], axis=1)
    rhs = xt @ R.astype(np.float64).T
    err = rel_l2(lhs, rhs)
    assert err <= 1e-12, err


def check_split_hand(split):
    g = golden_io.matrices("split_hand.txt")
    U, W = split(g["R"].astype(np.float32))
    assert np.array_equal(U.real, g["ReU"]) and np.array_equal(U.imag, g["ImU"])
    assert np.array_equal(W.real, g["ReW"]) and np.array_equal(W.imag, g["ImW"])
    m = U.shape[1]
    xt = g["x"][0]
    x = xt[:m] + 1j * xt[m:]
    y = U @ x + W @ np.conj(x)
    assert np.array_equal(np.concatenate([y.real, y.imag]), g["y"][0])


def check_split_unique(split):
    """The map R -> (U, W) is linear and invertible: the 4x4 matrix that sends one
    block entry (A, B, C, D) to (ReU, ImU, ReW, ImW) has full rank ("lossless and unique")."""
    cols = []
    for e in np.eye(4):
        R = np.array([[e[0], e[1]], [e[2], e[3]]], dtype=np.float32)
        U, W = split(R)
        cols.append([U[0, 0].real, U[0, 0].imag, W[0, 0].real, W[0, 0].imag])
    Mx = np.array(cols).T
    assert np.linalg.matrix_rank(Mx) == 4


# ----------------------------------------------------------- projection ----

def _brute_code(w: complex) -> int:
    scores = [(w * s.conjugate()).real for s in CODEWORDS]
    best = max(scores)
    return scores.index(best)          # first codeword in order 1, i, -1, -i


def check_project_bruteforce(project):
    """Every w = a + ib with a, b in a grid of small integers (all ties included)."""
    vals = [-3, -2, -1, -0.0, 0, 1, 2, 3]
    pts = list(itertools.product(vals, vals))
    a = np.array([p[0] for p in pts], dtype=np.float64)
    b = np.array([p[1] for p in pts], dtype=np.float64)
    k = project(a, b)
    want = [_brute_code(complex(x, y)) for x, y in pts]
    assert list(map(int, k)) == want


def check_project_angle(project, seed=1, count=20000):
    """Away from ties the code is the codeword nearest by angle (ModelScope card, "Method")."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(count)
    b = rng.standard_normal(count)
    k = project(a, b)
    for i in range(count):
        th = cmath.phase(complex(a[i], b[i]))
        d = [abs((th - cmath.phase(s) + math.pi) % (2 * math.pi) - math.pi) for s in CODEWORDS]
        assert int(k[i]) == int(np.argmin(d))


def check_project_golden(project):
    cases = golden_io.projection_cases()
    a = np.array([c[0] for c in cases])
    b = np.array([c[1] for c in cases])
    k = project(a, b)
    assert list(map(int, k)) == [c[2] for c in cases]


# ------------------------------------------------------------- ordered sum ----

def check_ordered_sum_golden(ordered_row_sum):
    for m, entries, want in golden_io.order_sum_cases():
        v = np.zeros((1, m))
        for j, val in entries.items():
            v[0, j] = val
        got = ordered_row_sum(v)[0]
        assert got == want, (m, got, want)


def check_ordered_sum_exact(ordered_row_sum, seed=2):
    """On small integers every order is exact: the result equals the integer sum."""
    rng = np.random.default_rng(seed)
    for m in (1, 64, 255, 256, 257, 2048, 5504):
        v = rng.integers(0, 1000, size=(3, m)).astype(np.float64)
        assert np.array_equal(ordered_row_sum(v), v.sum(axis=1))


# -------------------------------------------------------------- quantize ----

def _hand_row_R(unsplit, d):
    U = (d["U_re"] + 1j * d["U_im"])[None, :]
    W = (d["W_re"] + 1j * d["W_im"])[None, :]
    return unsplit(U, W)


def check_quantize_hand(quantize, unsplit):
    d = golden_io.quantize_hand()
    R = _hand_row_R(unsplit, d)
    codes, s32, s64, norms = quantize(R.astype(np.float32), 2)
    for (mat, t), want in d["codes"].items():
        M = 0 if mat == "U" else 1
        assert list(map(int, codes[t, M, 0])) == want, (mat, t)
    for (mat, t), (sre, sim) in d["scales"].items():
        M = 0 if mat == "U" else 1
        assert s64[0, t, M, 0] == sre and s64[0, t, M, 1] == sim, (mat, t)
    for mat, want in d["normsq"].items():
        M = 0 if mat == "U" else 1
        assert np.allclose(norms[M] ** 2, want, rtol=1e-15, atol=0), (mat, norms[M] ** 2, want)


def check_ls_identity(quantize, split, dequantize, seed=3, shape=(64, 256), T=3):
    """For each stage, ||r_t||^2 - ||r_{t+1}||^2 = sum_rows N_re s_re^2 + N_im s_im^2.

    This holds exactly in the reals exactly when s is the mean |component| over the
    entries assigned to that axis (the least-squares scale for fixed codes)."""
    rng = np.random.default_rng(seed)
    R = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    codes, s32, s64, norms = quantize(R, T)
    for M in range(2):
        for t in range(T):
            k = codes[t, M]
            n_re = ((k == 0) | (k == 2)).sum(axis=1)
            n_im = ((k == 1) | (k == 3)).sum(axis=1)
            drop = norms[M, t] ** 2 - norms[M, t + 1] ** 2
            want = float(np.sum(n_re * s64[:, t, M, 0] ** 2 + n_im * s64[:, t, M, 1] ** 2))
            assert abs(drop - want) <= 1e-12 * norms[M, 0] ** 2, (M, t, drop, want)
    # the final residual is the split minus the dequantized sum of all stages
    U, W = split(R)
    Uh, Wh = dequantize(codes, s64)
    for M, (Z, Zh) in enumerate(((U, Uh), (W, Wh))):
        assert abs(np.linalg.norm(Z - Zh) - norms[M, T]) <= 1e-12 * norms[M, 0]


def check_norm_nonincreasing(quantize, seed=4, shape=(128, 512), T=4):
    rng = np.random.default_rng(seed)
    R = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    _, _, _, norms = quantize(R, T)
    for M in range(2):
        assert np.all(np.diff(norms[M]) <= 0), norms[M]
        assert norms[M, 1] < norms[M, 0]


def check_codes_maximize_score(quantize, split, dequantize, seed=5, shape=(16, 64), T=2):
    """Each stage's code maximizes Re(r conj(s)) over the codebook for that stage's residual."""
    rng = np.random.default_rng(seed)
    R = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    codes, _, s64, _ = quantize(R, T)
    U, W = split(R)
    for M, Z in enumerate((U, W)):
        r = Z.copy()
        for t in range(T):
            for i in range(r.shape[0]):
                for j in range(r.shape[1]):
                    assert int(codes[t, M, i, j]) == _brute_code(complex(r[i, j]))
            one = np.zeros_like(codes[:1])
            one[0] = codes[t]
            hat = dequantize(one, s64[:, t:t + 1])[M]
            r = r - hat


def check_idempotent(quantize, unsplit, seed=6, n=8, m=64):
    """A row whose entries are already +-c or +-i c' (dyadic c, c') is recovered exactly by
    stage 0, and stage 1 then sees a zero residual: all codes 0, scales 0."""
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 4, size=(2, n, m))
    c_re = 2.0 ** rng.integers(-8, 0, size=(2, n))
    c_im = 2.0 ** rng.integers(-8, 0, size=(2, n))
    Z = []
    for M in range(2):
        z = np.zeros((n, m), dtype=np.complex128)
        z += np.where(k[M] == 0, 1, np.where(k[M] == 2, -1, 0)) * c_re[M][:, None]
        z += 1j * np.where(k[M] == 1, 1, np.where(k[M] == 3, -1, 0)) * c_im[M][:, None]
        # make sure both axes are used in every row
        z[:, 0] = c_re[M]
        z[:, 1] = 1j * c_im[M]
        Z.append(z)
    R = unsplit(Z[0], Z[1]).astype(np.float32)
    codes, _, s64, norms = quantize(R, 2)
    for M in range(2):
        kk = k[M].copy()
        kk[:, 0] = 0
        kk[:, 1] = 1
        assert np.array_equal(codes[0, M], kk)
        assert np.array_equal(s64[:, 0, M, 0], c_re[M]) and np.array_equal(s64[:, 0, M, 1], c_im[M])
        assert np.all(codes[1, M] == 0) and np.all(s64[:, 1, M] == 0)
        assert norms[M, 1] == 0.0


def check_empty_axis(quantize, unsplit):
    """A row with every entry on the real axis gets s_im = 0 (and vice versa)."""
    n, m = 2, 64
    U = np.zeros((n, m), dtype=np.complex128)
    U[0] = np.linspace(0.5, 1.0, m)           # all real, positive -> code 0
    U[1] = 1j * np.linspace(-1.0, -0.5, m)    # all imaginary, negative -> code 3
    W = U.copy()
    R = unsplit(U, W).astype(np.float32)
    codes, _, s64, _ = quantize(R, 1)
    assert np.all(codes[0, :, 0] == 0) and np.all(codes[0, :, 1] == 3)
    assert np.all(s64[0, 0, :, 1] == 0) and np.all(s64[0, 0, :, 0] > 0)
    assert np.all(s64[1, 0, :, 0] == 0) and np.all(s64[1, 0, :, 1] > 0)


# ----------------------------------------------------------------- pack ----

def check_pack_golden(pack_words):
    """Word encoding: 16 codes -> one little-endian 32-bit word, hand-worked bytes."""
    rows = golden_io.pack_bytes()
    codes = np.array([r[:16] for r in rows], dtype=np.uint8).reshape(1, 1, len(rows), 16)
    codes = np.concatenate([codes, codes], axis=1)           # U and W
    w = np.asarray(pack_words(codes))
    assert w.shape == (1, 2, len(rows), 1)
    for i, r in enumerate(rows):
        for M in range(2):
            b = [(int(w[0, M, i, 0]) >> (8 * k)) & 255 for k in range(4)]
            assert b == list(r[16:]), (i, M, b)


def check_pack_tile_order(pack, unpack):
    """Word order: a single nonzero code lands on the hand-worked byte and bit (n = 20,
    m = 320, T = 2: two row tiles, the second padded; a full and a one-group chunk)."""
    total, rows = golden_io.pack_tile_order()
    for t, M, i, j, off, sh in rows:
        for v in (1, 2, 3):
            codes = np.zeros((2, 2, 20, 320), dtype=np.uint8)
            codes[t, M, i, j] = v
            p = np.asarray(pack(codes))
            assert p.size == total
            nz = np.flatnonzero(p)
            assert list(nz) == [off], (t, M, i, j, list(nz[:4]))
            assert int(p[off]) == v << sh, (t, M, i, j, int(p[off]))
            assert np.array_equal(unpack(p, 20, 320, 2), codes)


def check_pack_roundtrip(pack, unpack, packed_nbytes, seed=7):
    rng = np.random.default_rng(seed)
    for T, n, m in ((1, 3, 64), (2, 5, 128), (3, 2, 320), (4, 17, 192), (2, 32, 1024), (1, 16, 256)):
        c = rng.integers(0, 4, size=(T, 2, n, m), dtype=np.uint8)
        p = pack(c)
        assert p.nbytes == packed_nbytes(n, m, T)
        assert np.array_equal(unpack(p, n, m, T), c)
        # padding rows of the last tile hold code 0: n rows of codes and nothing else is nonzero
        ones = pack(np.ones_like(c))
        assert int(np.unpackbits(ones).sum()) == T * 2 * n * m


def check_storage_bits(pack):
    """Packed bytes per real parameter of R equal the pages' bit budget."""
    for T, bits in golden_io.storage_bits():
        n, m = 16, 64
        p = pack(np.zeros((T, 2, n, m), dtype=np.uint8))
        real_params = (2 * n) * (2 * m)
        assert 8 * p.nbytes / real_params == bits


# ----------------------------------------------------------------- gemv ----

def _hand_gemv_inputs(d, T):
    codes = np.zeros((T, 2, 1, 2), dtype=np.uint8)
    scales = np.zeros((1, T, 2, 2))
    for t in range(T):
        for M, mat in enumerate("UW"):
            codes[t, M, 0] = d["codes"][(mat, t)]
            scales[0, t, M] = d["scales"][(mat, t)]
    return codes, scales


def check_gemv_hand(gemv_ref):
    d = golden_io.gemv_hand()
    for T in (1, 2):
        codes, scales = _hand_gemv_inputs(d, T)
        y = gemv_ref(codes, scales, d["x"][None, :])
        assert np.array_equal(y[0], d["y"][f"T{T}"]), (T, y)


def multiplication_free_gemv(codes, scales, x):
    """Python-loop GEMV that never multiplies a weight: each code adds or subtracts x_j,
    or swaps real and imaginary parts with a sign (zhichai.net note, "Industry
    implications"), into one accumulator per (stage, matrix, axis); the scale is applied
    once per accumulator.  Tiny shapes only."""
    T, _, n, m = codes.shape
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros((x.shape[0], 2 * n))
    for bi in range(x.shape[0]):
        a, b = x[bi, :m], x[bi, m:]
        for i in range(n):
            yr = yi = 0.0
            for t in range(T):
                for M in range(2):
                    acc = {0: [0.0, 0.0], 1: [0.0, 0.0]}     # axis -> complex accumulator
                    for j in range(m):
                        xr, xi = a[j], (b[j] if M == 0 else -b[j])    # W multiplies conj(x)
                        k = int(codes[t, M, i, j])
                        if k == 0:      # +1
                            acc[0][0] += xr; acc[0][1] += xi
                        elif k == 2:    # -1
                            acc[0][0] -= xr; acc[0][1] -= xi
                        elif k == 1:    # +i: (xr + i xi) i = -xi + i xr
                            acc[1][0] -= xi; acc[1][1] += xr
                        else:           # -i: xi - i xr
                            acc[1][0] += xi; acc[1][1] -= xr
                    s_re, s_im = float(scales[i, t, M, 0]), float(scales[i, t, M, 1])
                    yr += s_re * acc[0][0] + s_im * acc[1][0]
                    yi += s_re * acc[0][1] + s_im * acc[1][1]
            out[bi, i] = yr
            out[bi, n + i] = yi
    return out


def check_gemv_routes(gemv_ref, gemv_ref_real, seed=8, T=2, n=6, m=16, B=3):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 4, size=(T, 2, n, m), dtype=np.uint8)
    scales = rng.random((n, T, 2, 2)).astype(np.float32)
    x = rng.standard_normal((B, 2 * m))
    y1 = gemv_ref(codes, scales, x)
    assert rel_l2(y1, gemv_ref_real(codes, scales, x)) <= 1e-12
    assert rel_l2(y1, multiplication_free_gemv(codes, scales, x)) <= 1e-12
    # parallel stages: the stage terms are independent and summed
    ysum = sum(gemv_ref(codes, scales, x, stages=[t]) for t in range(T))
    assert rel_l2(y1, ysum) <= 1e-12


def check_gemv_lossless(gemv_ref, quantize, split, seed=9):
    """Dequantized layer applied to x equals R^ x~ where R^ is rebuilt from U^, W^:
    with T large the quantized map converges to R's map (residual shrinks)."""
    rng = np.random.default_rng(seed)
    R = (rng.standard_normal((32, 64)) * 0.02).astype(np.float32)
    x = rng.standard_normal((2, 64))
    exact = x @ R.astype(np.float64).T
    errs = []
    for T in (1, 2, 4, 8):
        codes, s32, s64, _ = quantize(R, T)
        errs.append(rel_l2(gemv_ref(codes, s64, x), exact))
    assert all(e2 < e1 for e1, e2 in zip(errs, errs[1:])), errs


# -------------------------------------------------------------- prefill ----

def check_act_quant_golden(act_quant_ref):
    toks = golden_io.act_quant_hand()
    x = np.stack([t["x"] for t in toks])
    q, delta = act_quant_ref(x)
    for i, t in enumerate(toks):
        assert [int(v) for v in q[i]] == [int(v) for v in t["q"]], i
        assert float(delta[i]) == t["delta"]


def check_act_quant_props(act_quant_ref, seed=10):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((64, 256)).astype(np.float32).astype(np.float64)
    q, delta = act_quant_ref(x)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    amax_idx = np.argmax(np.abs(x), axis=1)
    for i in range(x.shape[0]):
        assert abs(int(q[i, amax_idx[i]])) == 127
        assert int(np.sign(q[i, amax_idx[i]])) == int(np.sign(x[i, amax_idx[i]]))
        # |q - x/delta| <= 1/2 (+ the fp32 rounding of the ratio)
        assert np.all(np.abs(q[i] - x[i] / float(delta[i])) <= 0.5 + 1e-4)
        assert float(delta[i]) == float(np.float32(np.max(np.abs(x[i])) / 127.0))


def check_gemm_routes(gemm_int_ref, gemm_int_ref_loops, seed=11, T=2, n=3, m=8, N=4):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 4, size=(T, 2, n, m), dtype=np.uint8)
    q = rng.integers(-127, 128, size=(N, 2 * m)).astype(np.int8)
    assert np.array_equal(gemm_int_ref(codes, q), gemm_int_ref_loops(codes, q))


def check_gemm_epilogue(gemm_int_ref, gemm_epilogue_ref, gemv_ref, seed=12, T=3, n=5, m=32, N=6):
    """The prefill result is the GEMV of delta*q: both routes agree to 1e-12."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 4, size=(T, 2, n, m), dtype=np.uint8)
    scales = rng.random((n, T, 2, 2)).astype(np.float32)
    q = rng.integers(-127, 128, size=(N, 2 * m)).astype(np.int8)
    delta = (rng.random(N) * 0.05).astype(np.float32)
    y1 = gemm_epilogue_ref(gemm_int_ref(codes, q), scales, delta)
    y2 = gemv_ref(codes, scales, q.astype(np.float64) * delta.astype(np.float64)[:, None])
    assert rel_l2(y1, y2) <= 1e-12


def check_dequantize_real(dequantize_real, gemv_ref, seed=12, T=3, n=5, m=32, B=2):
    """The real form applied to x~ is the multiplication-free GEMV (a different route: per-code
    adds and swaps), and a single code with unit scales lands on the hand-derived blocks."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 4, size=(T, 2, n, m), dtype=np.uint8)
    scales = rng.random((n, T, 2, 2)).astype(np.float32)
    x = rng.standard_normal((B, 2 * m))
    R = dequantize_real(codes, scales)
    assert R.shape == (2 * n, 2 * m)
    assert rel_l2(x @ R.T, gemv_ref(codes, scales, x)) <= 1e-12
    # U has code 1 (= i, scale s_im = 3) at (0, 0), W code 2 (= -1, scale s_re = 5), T = 1:
    # U^ = 3i, W^ = -5 -> R11 = 0 + (-5), R12 = 0 - 3, R21 = 3 + 0, R22 = 0 - (-5)
    c = np.zeros((1, 2, 1, 1), dtype=np.uint8)
    c[0, 0, 0, 0], c[0, 1, 0, 0] = 1, 2
    s = np.zeros((1, 1, 2, 2))
    s[0, 0, 0, 1], s[0, 0, 1, 0] = 3.0, 5.0
    assert np.array_equal(dequantize_real(c, s), np.array([[-5.0, -3.0], [3.0, 5.0]]))


def check_per_tensor_scales(quantize, split, seed=21, T=2):
    """Per-tensor scales: (i) a one-row matrix gives the per-row result; (ii) every row carries
    the same pair; (iii) for the final codes each pair minimises the whole matrix's squared
    error on its axis (the least-squares scale is the mean |component| over the coded entries);
    (iv) a hand-worked 2 x 1 case."""
    rng = np.random.default_rng(seed)
    R1 = (rng.standard_normal((2, 128)) * 0.02).astype(np.float32)
    a = quantize(R1, T, per_tensor=True)
    b = quantize(R1, T)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    R = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    codes, s32, s64, _ = quantize(R, T, per_tensor=True)
    assert np.all(s64 == s64[:1])
    U, W = split(R)
    for M, Z in enumerate((U, W)):
        r = Z.copy()
        for t in range(T):
            k = codes[t, M].astype(np.int64)
            on_re = (k == 0) | (k == 2)
            s_re, s_im = s64[0, t, M]
            # d/ds sum over re-axis entries of (|Re r| - s)^2 = 0  <=>  s = mean |Re r|
            if on_re.any():
                assert abs(np.mean(np.abs(r.real[on_re])) - s_re) <= 1e-15 * max(1.0, abs(s_re)) + 1e-18
            if (~on_re).any():
                assert abs(np.mean(np.abs(r.imag[~on_re])) - s_im) <= 1e-15 * max(1.0, abs(s_im)) + 1e-18
            b_re = np.where(k == 0, 1.0, np.where(k == 2, -1.0, 0.0))
            b_im = np.where(k == 1, 1.0, np.where(k == 3, -1.0, 0.0))
            r = r - (s_re * b_re + 1j * s_im * b_im)
    # hand-worked: a 4 x 2 R whose split is U = [2, 4]^T (one column, both entries on the real
    # axis) and W = 0.  Per row the scales are 2 and 4; per tensor both rows get (2 + 4) / 2 = 3.
    Rh = np.zeros((4, 2), dtype=np.float32)
    Rh[0, 0] = Rh[2, 1] = 2.0          # row 0: ReU = 2 (R11 = 2, R22 = 2)
    Rh[1, 0] = Rh[3, 1] = 4.0          # row 1: ReU = 4
    codes, _, s64, _ = quantize(Rh, 1, per_tensor=True)
    assert np.all(codes[0, 0] == 0) and s64[0, 0, 0, 0] == 3.0 and s64[1, 0, 0, 0] == 3.0
    codes, _, s64, _ = quantize(Rh, 1)
    assert s64[0, 0, 0, 0] == 2.0 and s64[1, 0, 0, 0] == 4.0


def check_per_tensor_order(quantize):
    """The per-tensor scale combines its row sums in the pinned order (hand-worked cases in
    tests/golden/tensor_order.txt, where a plain left-to-right or adjacent-pair order gives a
    different fp64 value)."""
    for n, rows, want in golden_io.tensor_order_cases():
        R = np.zeros((2 * n, 2), dtype=np.float32)
        for i, v in rows.items():
            R[i, 0] = v            # R11 = Re U + Re W
            R[n + i, 1] = v        # R22 = Re U - Re W  -> Re U = v, W = 0
        codes, _, s64, _ = quantize(R, 1, per_tensor=True)
        assert np.all(codes == 0)
        assert s64[0, 0, 0, 0] == want, (n, s64[0, 0, 0, 0], want)
        assert np.all(s64[:, 0, 0, 1] == 0.0) and np.all(s64[:, 0, 1] == 0.0)

