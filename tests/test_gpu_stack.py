"""GPU parity of the decode step over a layer stack (grouped launches per shared input, the
launch configuration bench.py times for the full 32-layer stack) on a 2-layer LLaMA-2-7B-shaped
stack: every projection's output against the oracle GEMV on sampled rows, eager and replayed
from a HIP graph."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2
from widely_linear_gemv_amd.stack import DecodeStep, GROUPS, PROJECTIONS

pytestmark = pytest.mark.gpu
T = 2


def build(dev, layers, B):
    host, dev_layers, xs, acts = [], [], [], []
    for L in range(layers):
        hl, dl = [], []
        for p, (_, rows, cols, _) in enumerate(PROJECTIONS):
            n, m = rows // 2, cols // 2
            codes = workloads.random_codes(T, n, m, seed=workloads.stack_layer(L, p).seed)
            scales = workloads.random_scales(n, T, seed=workloads.stack_layer(L, p).seed + 1)
            hl.append((codes, scales))
            dl.append((f2.fairy2i_pack(up(codes, dev)), up(scales, dev)))
        host.append(hl)
        dev_layers.append(dl)
        lx, la = [], []
        for g in range(GROUPS):
            cols = next(c for (_, _, c, grp) in PROJECTIONS if grp == g)
            a = workloads.activations(B, cols, workloads.stack_x_seed(L, g))
            la.append(a)
            lx.append(x_to_dev(a, dev))
        xs.append(lx)
        acts.append(la)
    return host, dev_layers, xs, acts


def check(host, acts, ys, label):
    rng = np.random.default_rng(5)
    for L, hl in enumerate(host):
        for p, (codes, scales) in enumerate(hl):
            n = codes.shape[2]
            rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 40, replace=False)]))
            want = oracle.gemv_ref(np.ascontiguousarray(codes[:, :, rows]), scales[rows],
                                   acts[L][PROJECTIONS[p][3]].values)
            got = down(ys[L][p])
            got = np.concatenate([got[:, rows], got[:, n + rows]], axis=1)
            assert rel_l2(got, want) <= TOL_F32, (label, L, PROJECTIONS[p][0])


@pytest.mark.parametrize("B,algo", [(1, None), (1, f2.GEMV_MFMA_F4), (2, f2.GEMV_MFMA_F4),
                                    (2, f2.GEMV_MFMA_I8), (8, None)],
                         ids=["b1-default", "b1-f4", "b2-f4", "b2-i8", "b8-default"])
def test_two_layer_stack(B, algo):
    """Default kernel (bf16 matrix cores on the bf16 x) and the digit-form kernels."""
    dev = device()
    host, dev_layers, xs, acts = build(dev, 2, B)
    step = DecodeStep(dev_layers, xs, algo=algo)
    announce("stack decode step B =", B, "algo", step.algo, "eager")
    check(host, acts, step.run(), f"eager B={B}")
    torch.cuda.synchronize()
    g = step.capture()
    for rep in range(2):
        for row in step.ys:
            for y in row:
                y.fill_(float("nan"))
        announce("stack decode step B =", B, "graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        check(host, acts, step.ys, f"graph B={B} replay {rep}")
