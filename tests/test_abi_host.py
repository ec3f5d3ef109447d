"""C-ABI checks that need no GPU: the library loads, exports every symbol the header declares,
and every argument error returns its documented status (checks run before any HIP call)."""
import ctypes
import os
import re

import pytest

import widely_linear_gemv_amd as f2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fairy2i.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(f2.LIB_PATH):
        from widely_linear_gemv_amd import build
        build.build()
    return f2.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fairy2i_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("fairy2i_quantize", "fairy2i_pack", "fairy2i_gemv", "fairy2i_gemm",
                 "fairy2i_act_quant", "fairy2i_last_error", "fairy2i_status_string"):
        assert want in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(f2.SIGNATURES)


def test_version_and_status_strings(L):
    assert f2.fairy2i_abi_version() == 7
    for s in range(8):
        assert f2.fairy2i_status_string(s) not in ("", "unknown status")
    assert f2.fairy2i_status_string(99) == "unknown status"


FAKE = 1 << 20          # a 16-byte aligned, never dereferenced address
FAKE_ODD = FAKE + 2     # misaligned
NULL = None
S = None                # default stream


def last():
    return f2.fairy2i_last_error()


def test_quantize_errors(L):
    q = L.fairy2i_quantize
    assert q(NULL, 256, 256, 2, FAKE, FAKE, NULL, NULL, S) == 1
    assert q(FAKE, 256, 256, 0, FAKE, FAKE, NULL, NULL, S) == 3
    assert q(FAKE, 256, 256, 5, FAKE, FAKE, NULL, NULL, S) == 3
    assert q(FAKE, 255, 256, 2, FAKE, FAKE, NULL, NULL, S) == 2
    assert q(FAKE, 256, 200, 2, FAKE, FAKE, NULL, NULL, S) == 2         # m = 100
    assert q(FAKE, 256, 2 * 16384 + 128, 2, FAKE, FAKE, NULL, NULL, S) == 2   # 2*T*m too big
    assert "65536" in last()
    assert q(FAKE, 256, 256, 2, FAKE_ODD, FAKE, NULL, NULL, S) == 5
    assert q(FAKE, 256, 256, 2, FAKE, FAKE, FAKE + 4, NULL, S) == 5     # scales64 needs 8


def test_quantize_bf16_errors(L):
    q = L.fairy2i_quantize_bf16
    assert q(NULL, 256, 256, 2, FAKE, FAKE, NULL, NULL, S) == 1
    assert q(FAKE, 256, 256, 5, FAKE, FAKE, NULL, NULL, S) == 3
    assert q(FAKE, 255, 256, 2, FAKE, FAKE, NULL, NULL, S) == 2
    assert q(FAKE + 1, 256, 256, 2, FAKE, FAKE, NULL, NULL, S) == 5


def test_quantize_row_launch_bound(L):
    # one workgroup per row: more than 2^24 - 16 rows is a shape error for every row kernel
    big = 2 * ((1 << 24) + 16)
    assert L.fairy2i_quantize(FAKE, big, 256, 2, FAKE, FAKE, NULL, NULL, S) == 2
    assert "at most" in last()
    assert L.fairy2i_dequantize(FAKE, FAKE, big // 2, 128, 2, FAKE, 0, S) == 2


def _ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_quantize_grouped_errors(L):
    q = L.fairy2i_quantize_grouped
    R, P, Sc = _ptrs(FAKE, FAKE), _ptrs(FAKE, FAKE), _ptrs(FAKE, FAKE)
    assert q(0, NULL, 0, 256, 256, 2, NULL, NULL, NULL, NULL, S) == 0            # nothing to do
    assert q(-1, R, 0, 256, 256, 2, P, Sc, NULL, NULL, S) == 2
    assert q(2, NULL, 0, 256, 256, 2, P, Sc, NULL, NULL, S) == 1
    assert q(2, R, 7, 256, 256, 2, P, Sc, NULL, NULL, S) == 4                     # R dtype
    assert q(2, R, 0, 256, 256, 5, P, Sc, NULL, NULL, S) == 3
    assert q(2, R, 0, 255, 256, 2, P, Sc, NULL, NULL, S) == 2
    assert q(2, R, 0, 256, 2 * 16384 + 128, 2, P, Sc, NULL, NULL, S) == 2          # 2*T*m too big
    assert q(2, R, 0, 2 * (1 << 23), 256, 2, P, Sc, NULL, NULL, S) == 2            # 2 x 2^23 rows >= 2^24
    assert "workgroups" in last()
    assert q(2, _ptrs(FAKE, NULL), 0, 256, 256, 2, P, Sc, NULL, NULL, S) == 1      # a NULL entry
    assert "layer 1" in last()
    assert q(2, R, 0, 256, 256, 2, _ptrs(FAKE, FAKE_ODD), Sc, NULL, NULL, S) == 5
    assert q(2, _ptrs(FAKE, FAKE + 2), 0, 256, 256, 2, P, Sc, NULL, NULL, S) == 5  # fp32 R needs 4
    assert q(2, R, 0, 256, 256, 2, P, Sc, _ptrs(NULL, FAKE + 4), NULL, S) == 5     # scales64 needs 8
    assert q(2, R, 0, 256, 256, 2, P, Sc, NULL, _ptrs(FAKE + 8, NULL), S) == 5     # codes need 16


def test_quantize_tensor_workspace_bytes(L):
    w = L.fairy2i_quantize_tensor_workspace_bytes
    assert w(1, 64, 2) == 48 + 128
    assert w(2048, 2048, 2) == 40 * 2048 + 128
    assert w(5, 64, 1) == 208 + 128          # 200 rounded up to 16
    assert w(0, 64, 2) == 0 and w(-3, 64, 2) == 0


def test_quantize_tensor_errors(L):
    q = L.fairy2i_quantize_tensor
    ws = 1 << 20

    def call(R=FAKE, dt=f2.F32, two_n=256, two_m=256, T=2, w=FAKE, wb=ws, packed=FAKE, sc=FAKE):
        return q(R, dt, two_n, two_m, T, w, wb, packed, sc, NULL, NULL, S)

    assert call(R=NULL) == 1 and call(w=NULL) == 1 and call(sc=NULL) == 1
    assert call(dt=f2.I8) == 4
    assert call(T=0) == 3
    assert call(two_n=255) == 2 and call(two_m=200) == 2
    assert call(two_m=2 * 32832) == 2                      # m > 32768
    assert call(wb=L.fairy2i_quantize_tensor_workspace_bytes(128, 128, 2) - 1) == 6
    assert call(R=FAKE + 2) == 5 and call(w=FAKE + 8) == 5
    assert call(R=FAKE + 2, dt=f2.BF16, w=FAKE + 8) == 5   # bf16 R may sit at 2 bytes; workspace not


def test_pack_errors(L):
    p = L.fairy2i_pack
    assert p(NULL, 4, 64, 2, FAKE, S) == 1
    assert p(FAKE, 4, 64, 9, FAKE, S) == 3
    assert p(FAKE, 0, 64, 2, FAKE, S) == 2
    assert p(FAKE, 4, 96, 2, FAKE, S) == 2
    assert p(FAKE, 4, 64, 2, FAKE_ODD, S) == 5


def test_gemv_errors(L):
    g = L.fairy2i_gemv
    ok = dict(packed=FAKE, scales=FAKE, n=8, m=64, T=2, x=FAKE, xd=f2.BF16, B=1, y=FAKE,
              yd=f2.F32, algo=f2.GEMV_VALU)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["packed"], a["scales"], a["n"], a["m"], a["T"], a["x"], a["xd"], a["B"], a["y"],
                 a["yd"], a["algo"], S)

    assert call(x=NULL) == 1
    assert call(xd=f2.I8) == 4
    assert call(yd=f2.I32) == 4
    assert call(algo=7) == 4 and call(algo=-1) == 4
    assert call(algo=f2.GEMV_MFMA, xd=f2.F32) == 4
    assert call(algo=f2.GEMV_MFMA_I8, xd=f2.F32) == 4
    assert call(algo=f2.GEMV_MFMA_I8, xd=f2.BF16) == 4         # needs the digit form
    assert "digit form" in last()
    assert call(algo=f2.GEMV_MFMA_I8, xd=f2.X_DIGITS, B=3) == 2
    assert call(algo=f2.GEMV_VALU, xd=f2.X_DIGITS) == 4
    assert call(algo=f2.GEMV_MFMA_BF16, xd=f2.X_DIGITS) == 4
    assert call(algo=f2.GEMV_MFMA_F4, xd=f2.X_DIGITS) == 4          # needs the fp6 form
    assert call(algo=f2.GEMV_MFMA_F4, xd=f2.F32) == 4               # bf16 x or the fp6 form
    assert call(algo=f2.GEMV_MFMA_F4, xd=f2.BF16, B=3, m=(1 << 19) + 64) == 2   # fp8 split: fp32 sums
    assert call(algo=f2.GEMV_MFMA_F4, xd=f2.BF16, m=8192 + 64) == 2    # records built in LDS
    assert call(algo=f2.GEMV_MFMA_F4, xd=f2.BF16, m=4096 + 64, B=2) == 2
    assert "fairy2i_x_digits_f6" in last()
    assert call(algo=f2.GEMV_MFMA_I8, xd=f2.X_DIGITS_F6) == 4
    assert call(algo=f2.GEMV_VALU, xd=f2.X_DIGITS_F6) == 4
    assert call(algo=f2.GEMV_MFMA_F4, xd=f2.X_DIGITS_F6, B=3) == 2
    assert call(algo=f2.GEMV_MFMA_F4, xd=f2.X_DIGITS_F6, m=(1 << 19) + 64) == 2   # fp32 sums exact
    assert call(algo=f2.GEMV_AUTO, xd=f2.X_DIGITS_F6, m=(1 << 19) + 64) == 2      # AUTO -> F4
    assert call(T=0) == 3
    assert call(B=0) == 2 and call(B=17) == 2
    assert call(m=32) == 2 and call(n=0) == 2
    assert call(x=FAKE_ODD) == 5
    assert call(y=FAKE + 8) == 5


def test_x_digits_f6_bytes_and_errors(L):
    b = L.fairy2i_x_digits_f6_bytes
    assert b(64, 1) == 64 + 4096 and b(2048, 1) == 64 + 8 * 4096 and b(320, 2) == 64 + 2 * 2 * 4096
    assert b(0, 1) == 0 and b(64, 0) == 0
    d = L.fairy2i_x_digits_f6
    assert d(NULL, f2.BF16, 64, 1, FAKE, S) == 1 and d(FAKE, f2.BF16, 64, 1, NULL, S) == 1
    assert d(FAKE, f2.I8, 64, 1, FAKE, S) == 4
    assert d(FAKE, f2.BF16, 96, 1, FAKE, S) == 2 and d(FAKE, f2.BF16, 64, 3, FAKE, S) == 2
    assert d(FAKE + 8, f2.BF16, 64, 1, FAKE, S) == 5 and d(FAKE, f2.F32, 64, 1, FAKE + 8, S) == 5


def test_packed_bytes(L):
    """Size of the packed form: whole 16-row tiles, T * 2 planes, m / 4 bytes per row and plane."""
    import oracle
    for n, m, T in ((1, 64, 1), (16, 64, 2), (17, 320, 2), (2048, 2048, 2), (5504, 4096, 3)):
        assert L.fairy2i_packed_bytes(n, m, T) == oracle.packed_nbytes(n, m, T)
    assert L.fairy2i_packed_bytes(0, 64, 2) == 0


def test_dequantize_errors(L):
    d = L.fairy2i_dequantize
    assert d(NULL, FAKE, 8, 64, 2, FAKE, f2.F32, S) == 1
    assert d(FAKE, FAKE, 8, 64, 2, NULL, f2.F32, S) == 1
    assert d(FAKE, FAKE, 8, 64, 2, FAKE, f2.I8, S) == 4
    assert d(FAKE, FAKE, 8, 64, 0, FAKE, f2.F32, S) == 3
    assert d(FAKE, FAKE, 8, 96, 2, FAKE, f2.F32, S) == 2
    assert d(FAKE, FAKE, 8, 64, 2, FAKE + 8, f2.BF16, S) == 5


def test_x_digits_errors(L):
    d = L.fairy2i_x_digits
    assert L.fairy2i_x_digits_bytes(2048, 1) == 64 + 8 * 2048
    assert L.fairy2i_x_digits_bytes(2048, 2) == 64 + 16 * 2048
    assert d(NULL, f2.BF16, 64, 1, FAKE, S) == 1
    assert d(FAKE, f2.BF16, 64, 1, NULL, S) == 1
    assert d(FAKE, f2.I8, 64, 1, FAKE, S) == 4
    assert d(FAKE, f2.BF16, 96, 1, FAKE, S) == 2
    assert d(FAKE, f2.BF16, 64, 3, FAKE, S) == 2 and d(FAKE, f2.BF16, 64, 0, FAKE, S) == 2
    assert d(FAKE_ODD, f2.BF16, 64, 1, FAKE, S) == 5
    assert d(FAKE, f2.BF16, 64, 1, FAKE + 4, S) == 5


def test_gemv_grouped_errors(L):
    g = L.fairy2i_gemv_grouped
    It = f2.GemvItem
    good = (It * 2)(It(FAKE, FAKE, FAKE, FAKE, 8), It(FAKE, FAKE, FAKE, FAKE, 24))
    assert g(None, 2, 64, 2, f2.BF16, 1, f2.F32, f2.GEMV_MFMA, S) == 1
    assert g(good, 0, 64, 2, f2.BF16, 1, f2.F32, f2.GEMV_MFMA, S) == 2
    bad = (It * 2)(It(FAKE, FAKE, FAKE, FAKE, 8), It(FAKE, None, FAKE, FAKE, 24))
    assert g(bad, 2, 64, 2, f2.BF16, 1, f2.F32, f2.GEMV_MFMA, S) == 1
    assert "item 1" in last()
    assert g(good, 2, 64, 2, f2.F32, 1, f2.F32, f2.GEMV_MFMA, S) == 4
    assert g(good, 2, 64, 0, f2.BF16, 1, f2.F32, f2.GEMV_MFMA, S) == 3
    assert g(good, 2, 96, 2, f2.BF16, 1, f2.F32, f2.GEMV_MFMA, S) == 2
    badn = (It * 1)(It(FAKE, FAKE, FAKE, FAKE, 0))
    assert g(badn, 1, 64, 2, f2.BF16, 1, f2.F32, f2.GEMV_MFMA, S) == 2
    odd = (It * 1)(It(FAKE, FAKE, FAKE_ODD, FAKE, 8))
    assert g(odd, 1, 64, 2, f2.BF16, 1, f2.F32, f2.GEMV_MFMA, S) == 5


def test_gemv_strided_errors(L):
    """Every call here fails its argument checks (no kernel is launched on these fake pointers)."""
    g = L.fairy2i_gemv_strided
    # (packed, pstride, scales, sstride, n, m, T, x, x_dtype, B, y, ystride, y_dtype, batch, algo, stream)
    args = [FAKE, 4096, FAKE, 64, 16, 64, 2, FAKE, f2.BF16, 1, FAKE, 64, f2.F32, 3, f2.GEMV_MFMA, S]

    def call(**kw):
        a = list(args)
        names = ["packed", "pstride", "scales", "sstride", "n", "m", "T", "x", "x_dtype", "B", "y",
                 "ystride", "y_dtype", "batch", "algo", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return g(*a)

    assert call(scales=None) == 1
    assert call(x_dtype=f2.F32) == 4                       # bf16 MFMA kernel takes bf16 x only
    assert call(T=5) == 3
    assert call(m=96) == 2
    assert call(batch=0) == 2 and "batch" in last()
    assert call(batch=(1 << 29) + 1, n=32) == 2            # batch * ceil(n/16) > 2^30
    assert call(pstride=-16) == 2
    assert call(ystride=16) == 2 and "overlap" in last()   # y rows of matrices overlap
    assert call(pstride=4104) == 5                         # not a multiple of 16
    assert call(ystride=66) == 5                           # 66 floats = 264 bytes
    assert call(packed=FAKE_ODD) == 5


def test_act_quant_errors(L):
    a = L.fairy2i_act_quant
    assert a(NULL, f2.BF16, 4, 128, FAKE, FAKE, S) == 1
    assert a(FAKE, f2.I8, 4, 128, FAKE, FAKE, S) == 4
    assert a(FAKE, f2.BF16, 0, 128, FAKE, FAKE, S) == 2
    assert a(FAKE, f2.BF16, 4, 12, FAKE, FAKE, S) == 2
    assert a(FAKE_ODD, f2.BF16, 4, 128, FAKE, FAKE, S) == 5


def test_gemm_errors(L):
    g = L.fairy2i_gemm
    base = [FAKE, FAKE, 8, 64, 2, FAKE, f2.I8, FAKE, 16, FAKE, f2.F32, NULL, 0, S]

    def call(idx_vals):
        a = list(base)
        for i, v in idx_vals.items():
            a[i] = v
        return g(*a)

    assert call({7: NULL}) == 1                   # int8 x needs delta
    assert call({6: f2.I32}) == 4
    assert call({10: f2.I8}) == 4
    assert call({4: 5}) == 3
    assert call({8: 0}) == 2
    assert call({3: 65}) == 2
    assert call({9: FAKE_ODD}) == 5
    need = L.fairy2i_gemm_workspace_bytes(8, 64, 2, 16, f2.BF16)
    assert need >= 16 * 128 + 16 * 4
    assert call({6: f2.BF16, 11: FAKE, 12: need - 1}) == 6
    assert L.fairy2i_gemm_workspace_bytes(8, 64, 2, 16, f2.I8) == 0


def test_python_binding_raises_with_message(L):
    import torch
    with pytest.raises(f2.Fairy2iError) as e:
        f2._check(L.fairy2i_pack(NULL, 4, 64, 2, FAKE, S))
    assert "ERR_NULL" in str(e.value) and "required" in str(e.value)
    assert torch is not None


def test_strided_binding_rejects_wrong_ranks():
    import torch
    packed = torch.zeros(2, 64, dtype=torch.uint8)
    scales = torch.zeros(2, 16, 2, 2, 2)
    x = torch.zeros(1, 32)
    with pytest.raises(ValueError):
        f2.fairy2i_gemv_strided(packed.flatten(), scales, x, torch.zeros(2, 1, 32))
    with pytest.raises(ValueError):
        f2.fairy2i_gemv_strided(packed, scales[0, 0], x, torch.zeros(2, 1, 32))
    with pytest.raises(ValueError):
        f2.fairy2i_gemv_strided(packed, scales, x, torch.zeros(2, 32))


def test_gemm_noalloc_errors(L):
    """Argument errors of the entry point that allocates nothing, all caught on the host; a call
    whose activation staging exceeds the static array is refused before any HIP call."""
    g = L.fairy2i_gemm_noalloc
    BF, F32, I8 = 1, 0, 2
    assert g(NULL, FAKE, 64, 256, 2, FAKE, BF, NULL, 8, FAKE, F32, S) == 1
    assert g(FAKE, FAKE, 64, 256, 2, FAKE, I8, NULL, 8, FAKE, F32, S) == 1     # int8 x needs delta
    assert g(FAKE, FAKE, 64, 256, 2, FAKE, 9, NULL, 8, FAKE, F32, S) == 4
    assert g(FAKE, FAKE, 64, 256, 2, FAKE, BF, NULL, 8, FAKE, 7, S) == 4
    assert g(FAKE, FAKE, 64, 256, 5, FAKE, BF, NULL, 8, FAKE, F32, S) == 3
    assert g(FAKE, FAKE, 64, 100, 2, FAKE, BF, NULL, 8, FAKE, F32, S) == 2
    assert g(FAKE, FAKE, 64, 256, 2, FAKE, BF, NULL, 0, FAKE, F32, S) == 2
    assert g(FAKE, FAKE, 64, 256, 2, FAKE_ODD, BF, NULL, 8, FAKE, F32, S) == 5
    limit = L.fairy2i_gemm_noalloc_max_bytes()
    assert limit == 32 << 20
    N = limit // (2 * 2048) + 1
    assert g(FAKE, FAKE, 64, 2048, 2, FAKE, BF, NULL, N, FAKE, F32, S) == 6
    assert "static scratch" in last()
