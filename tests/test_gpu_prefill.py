"""GPU parity: per-token int8 activations (bit-exact), the int8-MFMA GEMM's raw int32
accumulators (bit-exact) and its fp32 / bf16 outputs (relative L2 <= 1e-5 / 2e-3)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, check_bf16, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu


def edge_tokens(two_m):
    """All-zero token, exact half-way ratios (amax = 127 so delta = 1), +-amax, tiny values;
    ratios within a few fp32 steps of half-integers at a delta other than 1 (the kernel checks
    those with a true division); a row whose delta is subnormal."""
    t = np.zeros((6, two_m), dtype=np.float32)
    t[1, :8] = [127, -127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5]
    t[2, :] = 1e-3
    t[2, 5] = -4.0
    t[3, :] = np.linspace(-3, 3, two_m, dtype=np.float32)
    d = np.float32(np.float32(100.0) / np.float32(127.0))
    k = np.arange(two_m) % 253 - 126                          # half-integers k + 1/2, |k| <= 126
    near = (k + 0.5).astype(np.float32) * d                   # rounded products: x / d next to k + 1/2
    steps = (np.arange(two_m) % 5 - 2).astype(np.int32)       # -2 .. +2 fp32 steps away
    near = (near.view(np.int32) + steps).view(np.float32)
    t[4, :] = np.clip(near, -100.0, 100.0)
    t[4, 0] = 100.0                                           # amax = 100
    t[5, :] = np.linspace(-1e-39, 1e-39, two_m, dtype=np.float32)   # delta below 2^-120
    return t


def bf16_act(values):
    bits = workloads.f32_to_bf16_bits(values)
    return workloads.Activations(values=workloads.bf16_bits_to_f32(bits), dtype="bf16", bf16_bits=bits)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("two_m,N", [(4096, 2048), (128, 33), (2112, 17), (11008, 40), (20480, 9)])
def test_act_quant_bit_exact(dtype, two_m, N):
    """Token rows held in registers between the two passes (one to eight groups of 2048 values,
    partial last groups) and the re-reading form (rows longer than 16384)."""
    dev = device()
    base = workloads.activations(N, two_m, workloads.PREFILL_X_SEED + two_m, dtype).values
    vals = np.concatenate([base, edge_tokens(two_m)])
    act = bf16_act(vals) if dtype == "bf16" else workloads.Activations(values=vals, dtype="f32")
    announce("act_quant", dtype, vals.shape)
    q, d = f2.fairy2i_act_quant(x_to_dev(act, dev))
    q_ref, d_ref = oracle.act_quant_ref(act.values)
    assert np.array_equal(down(d).view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(down(q), q_ref)


def gemm_case(dev, codes, scales, act, tok_sample, label):
    T, _, n, m = codes.shape
    packed = up(oracle.pack(codes), dev)
    s = up(scales.astype(np.float32), dev)
    x = x_to_dev(act, dev)
    N = act.values.shape[0]
    q_ref, d_ref = oracle.act_quant_ref(act.values)
    sel = np.asarray(tok_sample)
    P_ref = oracle.gemm_int_ref(codes, q_ref[sel])
    # raw int32 (activations quantized inside from bf16)
    announce("gemm raw", label)
    delta = torch.empty(N, dtype=torch.float32, device=dev)
    P = down(f2.fairy2i_gemm(packed, s, x, x_scale=delta, y_dtype=torch.int32))
    assert P.shape == (T, 2, 2, 2, N, n)
    assert np.array_equal(P[:, :, :, :, sel, :], P_ref), label
    assert np.array_equal(down(delta).view(np.uint32), d_ref.view(np.uint32))
    # fp32 / bf16 epilogue
    want = oracle.gemm_epilogue_ref(P_ref, scales.astype(np.float32), d_ref[sel])
    announce("gemm", label, "f32 out")
    y = down(f2.fairy2i_gemm(packed, s, x, y_dtype=torch.float32))
    err = rel_l2(y[sel], want)
    assert err <= TOL_F32, (label, "f32", err)
    announce("gemm", label, "bf16 out")
    y = down(f2.fairy2i_gemm(packed, s, x, y_dtype=torch.bfloat16))
    check_bf16(y[sel], want, label)
    # pre-quantized int8 input gives the same raw result
    announce("gemm int8 input", label)
    P8 = down(f2.fairy2i_gemm(packed, s, up(q_ref, dev), x_scale=up(d_ref, dev), y_dtype=torch.int32))
    assert np.array_equal(P8[:, :, :, :, sel, :], P_ref)


@pytest.mark.parametrize("li", [0, 1], ids=["4096x4096", "11008x4096"])
def test_prefill_full_size(li):
    dev = device()
    layer = workloads.PREFILL_LAYERS[li]
    n, m = layer.n, layer.m
    T = 2
    codes = workloads.random_codes(T, n, m, seed=layer.seed)
    scales = workloads.random_scales(n, T, seed=layer.seed + 1)
    act = workloads.activations(workloads.PREFILL_TOKENS, 2 * m, workloads.PREFILL_X_SEED)
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([[0, 1, 2047], rng.choice(2048, 45, replace=False)]))
    gemm_case(dev, codes, scales, act, sample, layer.name)


def test_prefill_quantized_attention_layer():
    """Codes and scales from the oracle quantizer of the 4096x4096 layer."""
    dev = device()
    codes, s32, _, _ = oracle.quantize(workloads.PREFILL_LAYERS[0].weight(), 2)
    act = workloads.activations(256, 4096, workloads.PREFILL_X_SEED)
    gemm_case(dev, codes, s32, act, np.arange(256), "quantized 4096x4096, 256 tokens")


@pytest.mark.parametrize("n,m,T,N", [(1, 64, 1, 1), (17, 192, 2, 7), (33, 128, 3, 40), (5, 320, 4, 33),
                                     (48, 256, 2, 64), (20, 448, 1, 65), (100, 320, 3, 300),
                                     (300, 256, 2, 70)])
def test_prefill_ragged(n, m, T, N):
    """Ragged rows (workgroups of 8 tiles with absent tiles), columns (a partial 256-column
    chunk), tokens (a partial token block), every T, and edge activations."""
    dev = device()
    codes = workloads.random_codes(T, n, m, seed=n + m + N)
    scales = workloads.random_scales(n, T, seed=T + N)
    vals = workloads.activations(N, 2 * m, seed=N + 3).values
    if N >= 4:
        k = min(N, 6)
        vals[:k] = edge_tokens(2 * m)[:k]
    gemm_case(dev, codes, scales, bf16_act(vals), np.arange(N), f"n={n} m={m} T={T} N={N}")
