"""GPU parity: fairy2i_dequantize (the real form of a packed layer) against the oracle.

fp32 output: every element within 2^-20 of the row's scale magnitude sum (the kernel adds at
most 2T fp32 terms in stage order; the oracle sums in fp64); bf16 output: additionally one bf16
rounding.  A third route: the GEMV of the GPU's real form equals the GPU decode GEMV."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu


def bound(scales):
    """Per output row of R^ (2n rows): sum over stages and matrices of |s_re| + |s_im|."""
    s = np.abs(np.asarray(scales, dtype=np.float64)).sum(axis=(1, 2, 3))
    return np.concatenate([s, s])[:, None]


def check(dev, codes, scales, label):
    T, _, n, m = codes.shape
    want = oracle.dequantize_real(codes, scales)
    packed = up(oracle.pack(codes), dev)
    s = up(scales.astype(np.float32), dev)
    announce("dequantize", label, "f32")
    got = down(f2.fairy2i_dequantize(packed, s, m)).astype(np.float64)
    tol = 2.0 ** -20 * bound(scales)
    assert np.all(np.abs(got - want) <= tol), (label, float(np.max(np.abs(got - want) - tol)))
    announce("dequantize", label, "bf16")
    gb = down(f2.fairy2i_dequantize(packed, s, m, R_dtype=torch.bfloat16).float()).astype(np.float64)
    assert np.all(np.abs(gb - want) <= 2.0 ** -8 * np.abs(want) + tol), label
    return packed, s, got


def test_attention_layer_and_third_route():
    dev = device()
    codes, s32, _, _ = oracle.quantize(workloads.ATTN.weight(), 2)
    packed, s, Rhat = check(dev, codes, s32, "4096x4096 T=2")
    act = workloads.activations(2, 4096, workloads.ATTN_X_SEEDS[1])
    x = x_to_dev(act, dev)
    y = down(f2.fairy2i_gemv(packed, s, f2.fairy2i_x_digits(x), algo=f2.GEMV_MFMA_I8))
    assert rel_l2(y, act.values.astype(np.float64) @ Rhat.T) <= TOL_F32


@pytest.mark.parametrize("n,m,T", [(1, 64, 1), (17, 320, 3), (33, 192, 4), (100, 2048, 2)])
def test_ragged(n, m, T):
    dev = device()
    codes = workloads.random_codes(T, n, m, seed=n + 7 * m + T)
    scales = workloads.random_scales(n, T, seed=n + m)
    check(dev, codes, scales, f"n={n} m={m} T={T}")
