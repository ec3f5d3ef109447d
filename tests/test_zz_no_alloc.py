"""The prefill GEMM entry point that allocates nothing (fairy2i_gemm_noalloc, for callers that
cannot allocate device memory) against fairy2i_gemm with a caller workspace: raw int32 sums, the
fp32 and bf16 outputs and the per-token deltas bit for bit on two calls in a row (the second
smaller, so it runs over the first call's leftovers in the static array), the int32 sums also
against the oracle; int8 activations (no staging); and the size limit rejected on the host."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import announce, device, down, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu


def layer(n, m, T, seed):
    codes = workloads.random_codes(T, n, m, seed=seed)
    scales = workloads.random_scales(n, T, seed=seed + 1)
    return codes, scales


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call(x_dtype):
    dev = device()
    T = 2
    for n, m, N, seed in ((300, 512, 64, 71), (37, 256, 17, 72)):      # second call smaller
        codes, scales = layer(n, m, T, seed)
        packed, s = up(oracle.pack(codes), dev), up(scales, dev)
        act = workloads.activations(N, 2 * m, seed + 10, x_dtype)
        x = x_to_dev(act, dev)
        for y_dtype in (torch.int32, torch.float32, torch.bfloat16):
            announce("gemm noalloc", n, m, T, N, x_dtype, y_dtype)
            shape = (T, 2, 2, 2, N, n) if y_dtype == torch.int32 else (N, 2 * n)
            d_ref = torch.empty(N, dtype=torch.float32, device=dev)
            d_got = torch.full((N,), float("nan"), dtype=torch.float32, device=dev)
            y_ref = f2.fairy2i_gemm(packed, s, x, x_scale=d_ref, y_dtype=y_dtype)
            y_got = torch.full(shape, 0x5A, dtype=y_dtype, device=dev) if y_dtype == torch.int32 \
                else torch.full(shape, float("nan"), dtype=y_dtype, device=dev)
            f2.fairy2i_gemm_noalloc(packed, s, x, x_scale=d_got, y=y_got)
            a, b = down(y_ref), down(y_got)
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (n, m, N, y_dtype)
            assert np.array_equal(down(d_ref).view(np.uint32), down(d_got).view(np.uint32))
            if y_dtype == torch.int32:
                q, _ = oracle.act_quant_ref(act.values)
                assert np.array_equal(b, oracle.gemm_int_ref(codes, q))
        # delta not requested: it is staged in the static array too
        y2 = torch.empty((N, 2 * n), dtype=torch.float32, device=dev)
        f2.fairy2i_gemm_noalloc(packed, s, x, y=y2)
        assert np.array_equal(down(y2).view(np.uint32), down(f2.fairy2i_gemm(packed, s, x)).view(np.uint32))


def test_noalloc_int8_activations_and_limit():
    dev = device()
    n, m, T, N = 40, 320, 3, 9
    codes, scales = layer(n, m, T, 73)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    act = workloads.activations(N, 2 * m, 74)
    q, d = oracle.act_quant_ref(act.values)
    qg, dg = up(q, dev), up(d, dev)
    announce("gemm noalloc int8 x")
    y = torch.empty((T, 2, 2, 2, N, n), dtype=torch.int32, device=dev)
    f2.fairy2i_gemm_noalloc(packed, s, qg, x_scale=dg, y=y)
    assert np.array_equal(down(y), oracle.gemm_int_ref(codes, q))
    # a call whose staging exceeds the static array is refused before any launch
    limit = f2.fairy2i_gemm_noalloc_max_bytes()
    m_big = 2048
    N_big = limit // (2 * m_big) + 1
    assert f2.fairy2i_gemm_workspace_bytes(n, m_big, T, N_big, f2.BF16) > limit
    L = f2.lib()
    st = L.fairy2i_gemm_noalloc(packed.data_ptr(), s.data_ptr(), n, m_big, T, qg.data_ptr(), f2.BF16, None,
                                N_big, y.data_ptr(), f2.F32, None)
    assert st == 6 and "static scratch" in f2.fairy2i_last_error()
