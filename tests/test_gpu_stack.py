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


@pytest.mark.parametrize("B,algo,given", [(1, None, False), (1, f2.GEMV_MFMA_F4, False), (2, f2.GEMV_MFMA_F4, False),
                                          (2, f2.GEMV_MFMA_I8, False), (8, None, False), (1, f2.GEMV_MFMA_F4, True),
                                          (1, f2.GEMV_MFMA_I8, True)],
                         ids=["b1-default", "b1-f4", "b2-f4", "b2-i8", "b8-default", "b1-f4-given", "b1-i8-given"])
def test_two_layer_stack(B, algo, given):
    """Default kernel (bf16 matrix cores on the bf16 x), the digit-form kernels with the digit
    passes in the step, and with the digit forms made once beforehand."""
    dev = device()
    host, dev_layers, xs, acts = build(dev, 2, B)
    step = DecodeStep(dev_layers, xs, algo=algo, digits_given=given)
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


SAMPLE_LAYERS = (0, 31)


@pytest.fixture(scope="module")
def stack_sample():
    """Layers 0 and 31 of the 32-layer LLaMA-2-7B stack exactly as bench.py draws them (pinned
    NumPy generator, seed 5000 + 7 L + p), quantized by the oracle at T = 2."""
    import concurrent.futures
    import os

    device()                               # skips before the host work when there is no GPU

    def one(key):
        R = workloads.stack_layer(*key).weight()
        return key, (R, oracle.quantize(R, T))

    keys = [(L, p) for L in SAMPLE_LAYERS for p in range(len(PROJECTIONS))]
    announce("oracle: quantizing the sampled stack layers on the host")
    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:   # numpy releases the GIL
        return dict(ex.map(one, keys))


@pytest.mark.parametrize("L", SAMPLE_LAYERS)
def test_stack_sample_quantize(stack_sample, L):
    """Every projection of the sampled stack layers: packed bytes and fp64 / fp32 scales bit for
    bit against the oracle."""
    dev = device()
    for p, (name, rows, cols, _) in enumerate(PROJECTIONS):
        R, (codes, s32, s64, _) = stack_sample[(L, p)]
        announce("stack quantize layer", L, name, rows, cols)
        out = f2.fairy2i_quantize(up(R, dev), T, want_scales64=True)
        assert np.array_equal(down(out["packed"]), oracle.pack(codes)), (L, name)
        assert np.array_equal(down(out["scales64"]).view(np.uint64), s64.view(np.uint64)), (L, name)
        assert np.array_equal(down(out["scales"]).view(np.uint32), s32.view(np.uint32)), (L, name)


@pytest.mark.parametrize("B", [1, 8])
def test_stack_sample_decode_step(stack_sample, B):
    """One decode step (the default kernels, eager and replayed from a HIP graph) over the two
    sampled stack layers, quantized on the GPU: every output row of every projection against the
    oracle GEMV on the oracle's own codes and scales."""
    dev = device()
    layers, xs, acts = [], [], []
    for L in SAMPLE_LAYERS:
        dl = []
        for p in range(len(PROJECTIONS)):
            R, _ = stack_sample[(L, p)]
            q = f2.fairy2i_quantize(up(R, dev), T)
            dl.append((q["packed"], q["scales"]))
        layers.append(dl)
        lx, la = [], []
        for g in range(GROUPS):
            cols = next(c for (_, _, c, grp) in PROJECTIONS if grp == g)
            a = workloads.activations(B, cols, workloads.stack_x_seed(L, g))
            la.append(a)
            lx.append(x_to_dev(a, dev))
        xs.append(lx)
        acts.append(la)
    import concurrent.futures
    import os

    def ref(kp):
        k, p = kp
        _, (codes, s32, _, _) = stack_sample[(SAMPLE_LAYERS[k], p)]
        return oracle.gemv_ref(codes, s32, acts[k][PROJECTIONS[p][3]].values)

    kps = [(k, p) for k in range(len(SAMPLE_LAYERS)) for p in range(len(PROJECTIONS))]
    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        refs = list(ex.map(ref, kps))
    want = [[refs[k * len(PROJECTIONS) + p] for p in range(len(PROJECTIONS))] for k in range(len(SAMPLE_LAYERS))]
    step = DecodeStep(layers, xs)
    announce("stack sample decode step B =", B, "eager")
    ys = step.run()
    for k, L in enumerate(SAMPLE_LAYERS):
        for p in range(len(PROJECTIONS)):
            assert rel_l2(down(ys[k][p]), want[k][p]) <= TOL_F32, ("eager", L, PROJECTIONS[p][0])
    g = step.capture()
    for row in step.ys:
        for y in row:
            y.fill_(float("nan"))
    announce("stack sample decode step B =", B, "graph replay")
    g.replay()
    torch.cuda.synchronize()
    for k, L in enumerate(SAMPLE_LAYERS):
        for p in range(len(PROJECTIONS)):
            assert rel_l2(down(step.ys[k][p]), want[k][p]) <= TOL_F32, ("graph", L, PROJECTIONS[p][0])
