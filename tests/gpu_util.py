"""Shared helpers for the GPU parity tests (marked `gpu`)."""
import os
import sys

import numpy as np
import pytest
import torch

import widely_linear_gemv_amd as f2


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(f2.LIB_PATH):
        from widely_linear_gemv_amd import build
        build.build()
    f2.lib()
    return torch.device("cuda:0")


def announce(*what):
    """Name the case before its GPU work, so a failure that kills the process is attributable."""
    print("[case]", *what, flush=True)
    sys.stdout.flush()


def up(a: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def up_bf16(bits: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def x_to_dev(act, dev):
    """workloads.Activations -> device tensor in its storage dtype."""
    if act.dtype == "bf16":
        return up_bf16(act.bf16_bits, dev)
    return up(act.values.astype(np.float32), dev)


def down(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


TOL_F32 = 1e-5      # fp32-output path, relative L2 against the fp64 oracle
TOL_BF16 = 2e-3     # bf16-output path, relative L2 (outputs of >= 2048 values)
BF16_HALF_ULP = 2.0 ** -8


def check_bf16(got, want, label):
    """bf16 outputs: every element within one bf16 rounding (2^-8 relative) of the fp64 value,
    plus the fp32 tolerance; and relative L2 <= 2e-3 over outputs large enough for that
    statistic to be stable (a handful of values can exceed it from rounding alone)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want ** 2)))
    bound = BF16_HALF_ULP * np.abs(want) + TOL_F32 * rms
    bad = np.abs(got - want) > bound
    assert not bad.any(), (label, int(bad.sum()), float(np.max(np.abs(got - want) - bound)))
    if want.size >= 2048:
        err = rel_l2(got, want)
        assert err <= TOL_BF16, (label, err)
