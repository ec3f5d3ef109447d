"""The path through the C ABI from a plain C program (tests/c_abi/driver.c: no Python, no torch
in the process that calls the library): quantize, the VALU and fp4 decode GEMVs and the int8
prefill GEMM on a ragged layer, compared with the oracle -- packed bytes, fp32 and fp64 scales,
activation scales and int32 accumulators bit for bit, GEMV outputs within the fp32 tolerance --
plus four documented argument errors returned by the same calls."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_F32, announce, rel_l2

from widely_linear_gemv_amd import build

pytestmark = pytest.mark.gpu


def driver():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(build.LIB):
        build.build()
    if not os.path.exists(build.C_DRIVER) or os.path.getmtime(build.C_DRIVER) < os.path.getmtime(build.C_DRIVER_SRC):
        build.build_c_driver()
    return build.C_DRIVER


@pytest.mark.parametrize("two_n,two_m,T,B,N", [(200, 1280, 2, 2, 37), (64, 128, 3, 1, 5)])
def test_c_program_matches_oracle(tmp_path, two_n, two_m, T, B, N):
    exe = driver()
    n, m = two_n // 2, two_m // 2
    rng = np.random.default_rng(two_n + two_m + T)
    R = (rng.standard_normal((two_n, two_m)) * 0.02).astype(np.float32)
    x = rng.standard_normal((B, two_m)).astype(np.float32)
    xp = rng.standard_normal((N, two_m)).astype(np.float32)
    for name, a in (("R.f32", R), ("x.f32", x), ("xp.f32", xp)):
        a.tofile(tmp_path / name)
    announce("C driver", two_n, two_m, T, B, N)
    res = subprocess.run([exe, str(tmp_path), str(two_n), str(two_m), str(T), str(B), str(N)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr

    codes, s32, s64, _ = oracle.quantize(R.astype(np.float64), T)
    packed = np.fromfile(tmp_path / "packed.u8", dtype=np.uint8)
    assert np.array_equal(packed, oracle.pack(codes))
    assert np.array_equal(np.fromfile(tmp_path / "scales.f32", dtype=np.float32).view(np.uint32),
                          s32.reshape(-1).view(np.uint32))
    assert np.array_equal(np.fromfile(tmp_path / "scales64.f64", dtype=np.float64).view(np.uint64),
                          s64.reshape(-1).view(np.uint64))

    want = oracle.gemv_ref(codes, s32, x)
    assert rel_l2(np.fromfile(tmp_path / "y_valu.f32", dtype=np.float32).reshape(B, two_n), want) <= TOL_F32
    if B <= 2:
        assert rel_l2(np.fromfile(tmp_path / "y_f4.f32", dtype=np.float32).reshape(B, two_n), want) <= TOL_F32

    q, delta = oracle.act_quant_ref(xp)
    assert np.array_equal(np.fromfile(tmp_path / "delta.f32", dtype=np.float32).view(np.uint32),
                          delta.view(np.uint32))
    P = np.fromfile(tmp_path / "p.i32", dtype=np.int32).reshape(T, 2, 2, 2, N, n)
    assert np.array_equal(P.astype(np.int64), oracle.gemm_int_ref(codes, q))
