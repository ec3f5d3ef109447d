"""GPU parity at the longest rows the library accepts: m = 2^22 complex columns for the
dequantizer, the prefill path and the int8, bf16 and VALU decode GEMVs, 2^19 for the fp4 decode
GEMV (its digit records are sized per 256-column chunk), and 2 T m = 65536 for the quantizer (a
row's codes are staged on chip; m = 32768 for per-tensor scales).  Row counts are small and
ragged; the cases exercise every kernel's offsets and counts at the limit, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, check_bf16, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu

M_MAX = 1 << 22
M_MAX_F4 = 1 << 19

_CODES = {}


def layer_codes(n, m, T):
    """Random codes and scales of an n x m layer (seeded; cached per shape)."""
    key = (n, m, T)
    if key not in _CODES:
        _CODES[key] = (workloads.random_codes(T, n, m, seed=n + m + T), workloads.random_scales(n, T, seed=m + T))
    return _CODES[key]


@pytest.mark.parametrize("T,m,per_tensor", [(1, 32768, False), (2, 16384, False), (4, 8192, False),
                                          (1, 32768, True)])
def test_quantize_longest_rows(T, m, per_tensor):
    """Three complex rows (a partial tile) at the longest row for T: codes, packed words and
    fp64 / fp32 scales bit for bit (each lane's partial sums run over m / 256 columns)."""
    dev = device()
    n = 3
    R = workloads.weight(2 * n, 2 * m, seed=501 + T)
    announce("quantize", n, m, T, "per-tensor" if per_tensor else "per-row")
    if per_tensor:
        out = f2.fairy2i_quantize_tensor(up(R, dev), T, want_scales64=True, want_codes=True)
    else:
        out = f2.fairy2i_quantize(up(R, dev), T, want_scales64=True, want_codes=True)
    got = {k: down(v) for k, v in out.items()}
    codes, s32, s64, _ = oracle.quantize(R, T, per_tensor=per_tensor)
    assert np.array_equal(got["codes"], codes)
    assert np.array_equal(got["packed"], oracle.pack(codes))
    assert np.array_equal(got["scales64"].view(np.uint64), s64.view(np.uint64))
    assert np.array_equal(got["scales"].view(np.uint32), s32.view(np.uint32))


def test_dequantize_longest_rows():
    """The real form of a 5-row layer of 2^22 columns within the fp32 rounding of its terms."""
    dev = device()
    n, m, T = 5, M_MAX, 2
    codes, scales = layer_codes(n, m, T)
    s32 = scales.astype(np.float32)
    want = oracle.dequantize_real(codes, s32)
    announce("dequantize", n, m, T)
    got = down(f2.fairy2i_dequantize(up(oracle.pack(codes), dev), up(s32, dev), m)).astype(np.float64)
    bound = np.abs(s32.astype(np.float64)).sum(axis=(1, 2, 3))       # per row: sum of its term magnitudes
    assert np.all(np.abs(got - want) <= 2.0 ** -20 * np.concatenate([bound, bound])[:, None])


@pytest.mark.parametrize("algo,m,B", [("f4", M_MAX_F4, 1), ("f4", M_MAX_F4, 2), ("i8", M_MAX, 1),
                                      ("i8", M_MAX, 2), ("bf16", M_MAX, 1), ("bf16", M_MAX, 3),
                                      ("bf16", M_MAX, 16), ("bf16", 8448, 2), ("valu", M_MAX, 1),
                                      ("valu", M_MAX, 5), ("valu", 8256, 1)])
def test_gemv_longest_rows(algo, m, B):
    """Decode GEMV of a 5-row layer at each kernel's longest row, held to the fp32 tolerance.
    The digit-form kernels (fp4, int8) sum exact integers; the bf16-operand and VALU kernels split
    long rows into 8192-column segments whose sums are applied to the scales and added to the
    outputs, so no fp32 sum runs over more than a few hundred terms in series."""
    dev = device()
    n, T = 5, 2
    codes, scales = layer_codes(n, m, T)
    s32 = scales.astype(np.float32)
    act = workloads.activations(B, 2 * m, seed=600 + B)
    want = oracle.gemv_ref(codes, s32, act.values)
    x = x_to_dev(act, dev)
    if algo == "i8":
        x = f2.fairy2i_x_digits(x)
    elif algo == "f4":
        x = f2.fairy2i_x_digits_f6(x)
    algos = {"f4": f2.GEMV_MFMA_F4, "i8": f2.GEMV_MFMA_I8, "bf16": f2.GEMV_MFMA_BF16, "valu": f2.GEMV_VALU}
    packed, s = up(oracle.pack(codes), dev), up(s32, dev)
    announce("gemv", algo, n, m, T, B)
    got = down(f2.fairy2i_gemv(packed, s, x, algo=algos[algo]))
    err = rel_l2(got, want)
    assert err <= TOL_F32, (algo, err)
    announce("gemv", algo, n, m, T, B, "bf16 out")
    check_bf16(down(f2.fairy2i_gemv(packed, s, x, algo=algos[algo], y_dtype=torch.bfloat16)), want, algo)


def test_prefill_longest_rows():
    """Activation quantization (rows of 2^23 values, the re-reading form) and the GEMM's raw int32
    sums (|P| <= 127 m < 2^31) bit for bit at m = 2^22, 17 rows (a partial tile), 5 tokens."""
    dev = device()
    n, m, T, N = 17, M_MAX, 2, 5
    codes, scales = layer_codes(n, m, T)
    act = workloads.activations(N, 2 * m, seed=700)
    q_ref, d_ref = oracle.act_quant_ref(act.values)
    P_ref = oracle.gemm_int_ref(codes, q_ref)
    announce("prefill", n, m, T, N)
    delta = torch.empty(N, dtype=torch.float32, device=dev)
    P = down(f2.fairy2i_gemm(up(oracle.pack(codes), dev), up(scales.astype(np.float32), dev), x_to_dev(act, dev),
                             x_scale=delta, y_dtype=torch.int32))
    assert np.array_equal(down(delta).view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(P, P_ref)


@pytest.mark.parametrize("B,m", [(1, 16640), (3, 8448), (16, 16640)])
def test_gemv_long_rows_large_launch(B, m):
    """Long rows in the large-launch forms of the bf16 GEMV (one wave per tile at B <= 2, the
    shared-x workgroups at B >= 3): one 16-row layer repeated 1536 times through the strided call
    with stride 0, so every matrix reads the same codes.  Each output flushes its sums at least
    once (rows of more than 32 chunks); all copies must agree bit for bit and match the oracle
    within the fp32 tolerance."""
    dev = device()
    n, T, batch = 16, 2, 1536
    codes, scales = layer_codes(n, m, T)
    s32 = scales.astype(np.float32)
    act = workloads.activations(B, 2 * m, seed=610 + B)
    want = oracle.gemv_ref(codes, s32, act.values)
    packed = up(oracle.pack(codes), dev)
    pool = packed.unsqueeze(0).expand(batch, -1)
    spool = up(s32, dev)
    y = torch.empty((batch, B, 2 * n), dtype=torch.float32, device=dev)
    announce("gemv bf16 long rows, strided", batch, n, m, T, B)
    got = down(f2.fairy2i_gemv_strided(pool, spool, x_to_dev(act, dev), y, algo=f2.GEMV_MFMA_BF16))
    assert np.array_equal(got, np.broadcast_to(got[:1], got.shape))
    assert rel_l2(got[0], want) <= TOL_F32
