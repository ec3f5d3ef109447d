"""GPU parity: fairy2i_quantize and fairy2i_pack against the oracle, bit for bit.

Codes, packed bytes and the fp64 scales must match exactly; the fp32 scales are their
round-to-nearest-even.  Full matrices are compared where the oracle finishes in seconds;
the LLaMA-2 MLP shapes are compared on a sample of complex rows (each row i depends only on
rows i and n+i of R, so the oracle runs on that sub-matrix)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu


def gpu_quantize(R, T, dev):
    out = f2.fairy2i_quantize(up(R, dev), T, want_scales64=True, want_codes=True)
    return {k: down(v) for k, v in out.items()}


def assert_rows_match(R, T, rows, got, label):
    n = R.shape[0] // 2
    rows = np.asarray(rows)
    sub = np.concatenate([R[rows], R[n + rows]], axis=0)
    codes, s32, s64, _ = oracle.quantize(sub, T)
    m = R.shape[1] // 2
    assert np.array_equal(got["codes"][:, :, rows], codes), label + ": codes"
    assert np.array_equal(oracle.unpack(got["packed"], n, m, T)[:, :, rows], codes), label + ": packed"
    assert np.array_equal(got["scales64"][rows].view(np.uint64), s64.view(np.uint64)), label + ": scales64"
    assert np.array_equal(got["scales"][rows].view(np.uint32), s32.view(np.uint32)), label + ": scales"


def test_tiny_full():
    dev = device()
    R = workloads.TINY.weight()
    announce("quantize tiny 256x256 T=2")
    got = gpu_quantize(R, 2, dev)
    assert_rows_match(R, 2, np.arange(128), got, "tiny")


def test_attention_full():
    dev = device()
    R = workloads.ATTN.weight()
    announce("quantize 4096x4096 T=2")
    got = gpu_quantize(R, 2, dev)
    codes, s32, s64, _ = oracle.quantize(R, 2)
    assert np.array_equal(got["codes"], codes)
    assert np.array_equal(got["packed"], oracle.pack(codes))
    assert np.array_equal(got["scales64"].view(np.uint64), s64.view(np.uint64))
    assert np.array_equal(got["scales"].view(np.uint32), s32.view(np.uint32))


@pytest.mark.parametrize("layer", [workloads.MLP_GATE_UP, workloads.MLP_DOWN], ids=["gate_up", "down"])
@pytest.mark.parametrize("T", [2, 3])
def test_mlp_sampled_rows(layer, T):
    dev = device()
    R = layer.weight()
    announce("quantize", layer.name, "T =", T)
    got = gpu_quantize(R, T, dev)
    n = layer.n
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, n - 1], rng.choice(n, 93, replace=False)]))
    assert_rows_match(R, T, rows, got, layer.name)
    # codes and packed agree everywhere (the packed bytes are the codes, four to a byte)
    assert np.array_equal(oracle.unpack(got["packed"], n, layer.m, T), got["codes"])


def constructed_edge_matrix(n, m, seed):
    """Dyadic R whose U and W rows hit every special case: exact ties |Re| = |Im|, zeros,
    all-real rows (empty imaginary axis), all-imaginary rows, rows already in the codebook
    times a per-row scale (exact recovery), and random dyadic rows."""
    rng = np.random.default_rng(seed)
    Z = []
    for M in range(2):
        a = rng.integers(-8, 9, size=(n, m)).astype(np.float64) / 8.0
        b = rng.integers(-8, 9, size=(n, m)).astype(np.float64) / 8.0
        tie = rng.random((n, m)) < 0.3
        b = np.where(tie, np.where(rng.random((n, m)) < 0.5, a, -a), b)
        zero = rng.random((n, m)) < 0.05
        a[zero] = 0.0
        b[zero] = 0.0
        z = a + 1j * b
        z[0] = np.abs(a[0]) + 0.125                 # every code 0: empty imaginary axis
        z[1 % n] = 1j * (-np.abs(b[1 % n]) - 0.25)  # every code 3: empty real axis
        if n > 2:
            k = rng.integers(0, 4, size=m)
            z[2] = np.where(k == 0, 0.5, np.where(k == 2, -0.5, np.where(k == 1, 0.25j, -0.25j)))
        if n > 3:
            z[3] = 0.0                              # all zero
        Z.append(z)
    return oracle.unsplit(Z[0], Z[1]).astype(np.float32)


@pytest.mark.parametrize("n,m,T", [(4, 64, 2), (7, 320, 3), (33, 512, 1), (5, 2048, 4),
                                   (9, 5504, 2), (3, 6208, 2), (2, 64, 4)])
def test_edge_cases(n, m, T):
    """Ties, zeros, empty axes, exact recovery, ragged m (not a multiple of 256), the
    register-resident and the re-reading (m > 6144) kernel variants, T = 1..4."""
    dev = device()
    R = constructed_edge_matrix(n, m, seed=n * 1000 + m + T)
    announce("quantize edge", n, m, T)
    got = gpu_quantize(R, T, dev)
    assert_rows_match(R, T, np.arange(n), got, f"edge n={n} m={m} T={T}")


def test_random_fp32_ragged():
    dev = device()
    R = workloads.weight(2 * 37, 2 * 704, seed=55)
    announce("quantize random 74x1408 T=3")
    got = gpu_quantize(R, 3, dev)
    assert_rows_match(R, 3, np.arange(37), got, "ragged")


@pytest.mark.parametrize("T,n,m", [(1, 3, 64), (2, 17, 128), (3, 5, 192), (4, 2, 1024), (2, 2048, 2048)])
def test_pack_matches_oracle(T, n, m):
    dev = device()
    codes = workloads.random_codes(T, n, m, seed=T * 100 + n)
    noisy = codes | (np.random.default_rng(1).integers(0, 64, size=codes.shape, dtype=np.uint8) << 2)
    announce("pack", T, n, m)
    got = down(f2.fairy2i_pack(up(noisy, dev)))
    assert np.array_equal(got, oracle.pack(codes))     # bits above the code are ignored


@pytest.mark.parametrize("T", [1, 2])
def test_bf16_weights(T):
    """A bf16 layer quantizes exactly like its fp32 widening (bit-exact codes and scales)."""
    dev = device()
    R = workloads.ATTN.weight()[:512, :1024]
    bits = workloads.f32_to_bf16_bits(R)
    Rw = workloads.bf16_bits_to_f32(bits)
    announce("quantize bf16 weights T =", T)
    out = f2.fairy2i_quantize(torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16), T,
                              want_scales64=True, want_codes=True)
    got = {k: down(v) for k, v in out.items()}
    codes, s32, s64, _ = oracle.quantize(Rw, T)
    assert np.array_equal(got["codes"], codes)
    assert np.array_equal(got["packed"], oracle.pack(codes))
    assert np.array_equal(got["scales64"].view(np.uint64), s64.view(np.uint64))
    assert np.array_equal(got["scales"].view(np.uint32), s32.view(np.uint32))


def gpu_quantize_tensor(R, T, dev, *, dirty=True, bf16_bits=None):
    n, m = R.shape[0] // 2, R.shape[1] // 2
    ws = torch.full((f2.fairy2i_quantize_tensor_workspace_bytes(n, m, T),), 0xA5, dtype=torch.uint8, device=dev)
    packed = torch.full((f2.fairy2i_packed_bytes(n, m, T),), 0xFF if dirty else 0, dtype=torch.uint8, device=dev)
    Rg = up(R, dev) if bf16_bits is None else torch.from_numpy(bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    out = f2.fairy2i_quantize_tensor(Rg, T, want_scales64=True, want_codes=True, workspace=ws, packed=packed)
    return {k: down(v) for k, v in out.items()}


def assert_tensor_match(R, T, got, label):
    codes, s32, s64, _ = oracle.quantize(R, T, per_tensor=True)
    assert np.array_equal(got["codes"], codes), label + ": codes"
    assert np.array_equal(got["packed"], oracle.pack(codes)), label + ": packed (padding rows zero)"
    assert np.array_equal(got["scales64"].view(np.uint64), s64.view(np.uint64)), label + ": scales64"
    assert np.array_equal(got["scales"].view(np.uint32), s32.view(np.uint32)), label + ": scales"


@pytest.mark.parametrize("n,m,T", [(4, 64, 2), (7, 320, 3), (33, 512, 1), (5, 2048, 4),
                                   (9, 5504, 2), (3, 6208, 2), (300, 256, 2), (1, 64, 1)])
def test_tensor_scales_edge_cases(n, m, T):
    """Per-tensor scales: ties, zeros, empty axes, ragged m and n (padding rows written as zero
    over a dirty buffer), the register-resident and re-reading kernel variants, T = 1..4, more
    than 256 rows (several row sums per lane of the combining step)."""
    dev = device()
    R = constructed_edge_matrix(n, m, seed=n * 1000 + m + T + 7)
    announce("quantize per-tensor edge", n, m, T)
    assert_tensor_match(R, T, gpu_quantize_tensor(R, T, dev), f"tensor n={n} m={m} T={T}")


def test_tensor_scales_attention():
    """The 4096 x 4096 attention layer with per-tensor scales, compared in full."""
    dev = device()
    R = workloads.ATTN.weight()
    announce("quantize per-tensor 4096x4096 T=2")
    assert_tensor_match(R, 2, gpu_quantize_tensor(R, 2, dev), "attention")


def test_tensor_scales_bf16_and_reuse():
    """bf16 weights quantize like their fp32 widening; a second call on the same (now used)
    workspace and a smaller matrix gives the fresh result."""
    dev = device()
    R = workloads.weight(2 * 600, 2 * 1024, seed=66)
    bits = workloads.f32_to_bf16_bits(R)
    announce("quantize per-tensor bf16 1200x2048 T=2")
    assert_tensor_match(workloads.bf16_bits_to_f32(bits), 2, gpu_quantize_tensor(R, 2, dev, bf16_bits=bits), "bf16")
    n, m, T = 600, 1024, 2
    ws = torch.empty((f2.fairy2i_quantize_tensor_workspace_bytes(n, m, T),), dtype=torch.uint8, device=dev)
    for rows in (600, 77):
        Rs = np.concatenate([R[:rows, :2 * 256], R[n:n + rows, :2 * 256]], axis=0)
        out = f2.fairy2i_quantize_tensor(up(Rs, dev), T, want_scales64=True, want_codes=True, workspace=ws)
        assert_tensor_match(Rs, T, {k: down(v) for k, v in out.items()}, f"reuse rows={rows}")


def test_tensor_scales_feed_gemv():
    """The per-tensor output is an ordinary packed layer: the int8 decode GEMV on it matches the
    oracle GEMV with the same scales (relative L2 <= 1e-5)."""
    dev = device()
    n, m, T = 96, 512, 2
    R = workloads.weight(2 * n, 2 * m, seed=67)
    out = f2.fairy2i_quantize_tensor(up(R, dev), T)
    act = workloads.activations(1, 2 * m, seed=68)
    announce("per-tensor layer into the int8 GEMV")
    xd = f2.fairy2i_x_digits(x_to_dev(act, dev))
    y = down(f2.fairy2i_gemv(out["packed"], out["scales"], xd, algo=f2.GEMV_MFMA_I8))
    codes, s32, _, _ = oracle.quantize(R, T, per_tensor=True)
    assert rel_l2(y, oracle.gemv_ref(codes, s32, act.values)) <= TOL_F32


@pytest.mark.parametrize("case", range(3))
def test_tensor_scales_order_cases(case):
    """The hand-worked order cases of tests/golden/tensor_order.txt, widened to m = 64 (the
    value in column 0, zeros elsewhere: the row sums are unchanged and the count is 64 n): the
    per-tensor fp64 scale must come out in the pinned combining order, bit for bit."""
    import golden_io
    dev = device()
    n, rows, _ = golden_io.tensor_order_cases()[case]
    m = 64
    R = np.zeros((2 * n, 2 * m), dtype=np.float32)
    for i, v in rows.items():
        R[i, 0] = v
        R[n + i, m] = v
    announce("quantize per-tensor order case", case, n)
    assert_tensor_match(R, 1, gpu_quantize_tensor(R, 1, dev), f"order case {case}")


@pytest.mark.parametrize("count,n,m,T,dtype", [(3, 40, 128, 2, torch.float32),      # ragged tiles, MAXC 1
                                               (5, 16, 2048, 3, torch.float32),     # MAXC 8
                                               (2, 33, 5504, 2, torch.bfloat16),    # MAXC 24
                                               (2, 17, 8192, 1, torch.float32),     # re-read form
                                               (35, 24, 256, 4, torch.float32)])    # two launches (32 + 3)
def test_grouped_matches_single(count, n, m, T, dtype):
    """fairy2i_quantize_grouped: every layer's codes, packed bytes (padding rows included) and
    fp32/fp64 scales equal its own fairy2i_quantize call bit for bit; the first and last layers
    also against the oracle."""
    dev = device()
    rng = np.random.default_rng(count * 1000 + n + m + T)
    Rs = [torch.from_numpy((rng.standard_normal((2 * n, 2 * m)) * 0.02).astype(np.float32)).to(dev).to(dtype)
          for _ in range(count)]
    announce("quantize grouped", count, n, m, T, dtype)
    got = f2.fairy2i_quantize_grouped(Rs, T, want_scales64=True, want_codes=True)
    assert len(got) == count
    for k, R in enumerate(Rs):
        one = f2.fairy2i_quantize(R, T, want_scales64=True, want_codes=True)
        for key in ("packed", "codes"):
            assert torch.equal(got[k][key], one[key]), (k, key)
        assert torch.equal(got[k]["scales"].view(torch.int32), one["scales"].view(torch.int32)), k
        assert torch.equal(got[k]["scales64"].view(torch.int64), one["scales64"].view(torch.int64)), k
    for k in (0, count - 1):
        Rk = down(Rs[k].float()).astype(np.float32)
        assert_rows_match(Rk, T, np.arange(n), {kk: down(v) for kk, v in got[k].items()}, f"grouped layer {k}")
