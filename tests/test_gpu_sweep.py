"""Seeded sweep of random shapes through every entry point, against the oracle.

Each case draws its shape from a fixed seed (rows n from 1 to ~700, so partial and single-row
tiles; m any multiple of 64, so partial 256-column chunks; T = 1..4; batch within each kernel's
limit), then checks: the quantizer's packed bytes and fp64 scales bit for bit; every applicable
decode kernel (VALU, bf16 MFMA, int8 and fp4 on their digit forms, fp4 on bf16 x) within the fp32
tolerance, in a single call, a grouped call with a second, differently shaped item sharing m, and
a strided batch of three copies; the prefill GEMM's int32 accumulators bit for bit.  The shapes
are the sweep's, the oracle's sizes stay small enough to finish in seconds."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu

CASES = 64


def shape(k):
    rng = np.random.default_rng(7000 + k)
    n = int(rng.integers(1, 700))
    m = 64 * int(rng.integers(1, 41))
    while n * m > 160_000:                       # keep the oracle quick
        n = max(1, n // 2)
    T = int(rng.integers(1, 5))
    B = int(rng.choice([1, 1, 2, 2, 3, 4, 5, 8, 16]))
    N = int(rng.integers(1, 70))
    return n, m, T, B, N


def kernels(B):
    ks = [("valu", f2.GEMV_VALU, None), ("bf16", f2.GEMV_MFMA_BF16, None)]
    if B <= 2:
        ks += [("i8", f2.GEMV_MFMA_I8, f2.fairy2i_x_digits), ("f4", f2.GEMV_MFMA_F4, f2.fairy2i_x_digits_f6),
               ("f4 on bf16 x", f2.GEMV_MFMA_F4, None)]
    else:
        ks += [("f4 on bf16 x split into fp8", f2.GEMV_MFMA_F4, None)]
    return ks


@pytest.mark.parametrize("k", range(CASES))
def test_random_shape(k):
    dev = device()
    n, m, T, B, N = shape(k)
    announce("sweep", k, "n", n, "m", m, "T", T, "B", B, "N", N)
    rng = np.random.default_rng(9000 + k)

    # quantizer on a random real layer
    R = (rng.standard_normal((2 * n, 2 * m)) * 0.02).astype(np.float32)
    q = f2.fairy2i_quantize(up(R, dev), T, want_scales64=True)
    codes, s32, s64, _ = oracle.quantize(R, T)
    assert np.array_equal(down(q["packed"]), oracle.pack(codes)), k
    assert np.array_equal(down(q["scales64"]).view(np.uint64), s64.view(np.uint64)), k

    # decode GEMVs on the quantized layer
    act = workloads.activations(B, 2 * m, seed=9500 + k)
    x = x_to_dev(act, dev)
    want = oracle.gemv_ref(codes, s32, act.values)
    n2 = int(rng.integers(1, 200))                 # a second item of another height, same m and T
    codes2 = workloads.random_codes(T, n2, m, seed=9600 + k)
    scales2 = workloads.random_scales(n2, T, seed=9700 + k)
    want2 = oracle.gemv_ref(codes2, scales2, act.values)
    p2, s2 = up(oracle.pack(codes2), dev), up(scales2, dev)
    pool = torch.stack([q["packed"]] * 3)          # strided batch: three copies back to back
    spool = torch.stack([q["scales"]] * 3)
    for name, algo, digits in kernels(B):
        xx = digits(x) if digits is not None else x
        got = down(f2.fairy2i_gemv(q["packed"], q["scales"], xx, algo=algo))
        assert rel_l2(got, want) <= TOL_F32, (k, name)
        ys = f2.fairy2i_gemv_grouped([(q["packed"], q["scales"], xx, torch.empty((B, 2 * n), device=dev)),
                                      (p2, s2, xx, torch.empty((B, 2 * n2), device=dev))], algo=algo)
        assert rel_l2(down(ys[0]), want) <= TOL_F32, (k, name, "grouped")
        assert rel_l2(down(ys[1]), want2) <= TOL_F32, (k, name, "grouped item 2")
        ystride = -(-2 * n * B // 4) * 4              # per-matrix outputs start on 16-byte boundaries
        yb = torch.empty(3 * ystride, device=dev).as_strided((3, B, 2 * n), (ystride, 2 * n, 1))
        f2.fairy2i_gemv_strided(pool, spool, xx, yb, algo=algo)
        for j in range(3):
            assert rel_l2(down(yb[j]), want) <= TOL_F32, (k, name, "strided", j)

    # prefill GEMM, raw accumulators
    xp = workloads.activations(N, 2 * m, seed=9800 + k)
    P = down(f2.fairy2i_gemm(q["packed"], q["scales"], x_to_dev(xp, dev), y_dtype=torch.int32))
    qq, _ = oracle.act_quant_ref(xp.values)
    assert np.array_equal(P.astype(np.int64), oracle.gemm_int_ref(codes, qq)), k
