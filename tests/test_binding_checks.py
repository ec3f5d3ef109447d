"""The Python binding checks every tensor before it hands a pointer to the C ABI (which takes no
buffer sizes): wrong dtype, shape, size, layout or device raises ValueError and launches nothing.
CPU only -- every tensor here lives on the CPU, so a call that got past the checks would reach the
library and fail there with a HIP error instead of a ValueError."""
import pytest
import torch

import widely_linear_gemv_amd as f2

n, m, T, B = 32, 128, 2, 2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(f2.LIB_PATH):
        from widely_linear_gemv_amd import build
        build.build()
    f2.lib()


def layer():
    return (torch.zeros(f2.fairy2i_packed_bytes(n, m, T), dtype=torch.uint8),
            torch.zeros((n, T, 2, 2), dtype=torch.float32))


def raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_quantize_checks():
    R = torch.zeros((2 * n, 2 * m), dtype=torch.float32)
    raises("dtype", f2.fairy2i_quantize, R.double(), T)
    raises("shape", f2.fairy2i_quantize, R[:-1], T)
    raises("contiguous", f2.fairy2i_quantize, R.t(), T)
    packed, scales = layer()
    raises("bytes", f2.fairy2i_quantize, R, T, packed=packed[:-16], scales=scales)
    raises("shape", f2.fairy2i_quantize, R, T, packed=packed, scales=scales[:-1])
    raises("dtype", f2.fairy2i_quantize, R, T, packed=packed, scales=scales.double())
    raises("GPU", f2.fairy2i_quantize, R, T)                       # everything else right


def test_quantize_grouped_checks():
    R = torch.zeros((2 * n, 2 * m), dtype=torch.float32)
    assert f2.fairy2i_quantize_grouped([], T) == []
    raises("group", f2.fairy2i_quantize_grouped, [R, R[:, :-2].contiguous()], T)     # another shape
    raises("group", f2.fairy2i_quantize_grouped, [R, R.bfloat16()], T)              # another dtype
    raises("dtype", f2.fairy2i_quantize_grouped, [R.double()], T)
    raises("contiguous", f2.fairy2i_quantize_grouped, [R, R.t()], T)
    packed, scales = layer()
    raises("outputs", f2.fairy2i_quantize_grouped, [R, R], T, packed=[packed])
    raises("bytes", f2.fairy2i_quantize_grouped, [R], T, packed=[packed[:-16]], scales=[scales])
    raises("GPU", f2.fairy2i_quantize_grouped, [R, R], T)                            # everything else right


def test_quantize_tensor_checks():
    R = torch.zeros((2 * n, 2 * m), dtype=torch.bfloat16)
    ws = torch.zeros(f2.fairy2i_quantize_tensor_workspace_bytes(n, m, T), dtype=torch.uint8)
    raises("bytes", f2.fairy2i_quantize_tensor, R, T, workspace=ws[:-16])
    raises("GPU", f2.fairy2i_quantize_tensor, R, T, workspace=ws)


def test_pack_and_dequantize_checks():
    codes = torch.zeros((T, 2, n, m), dtype=torch.uint8)
    raises("dtype", f2.fairy2i_pack, codes.int())
    raises("shape", f2.fairy2i_pack, codes[:, :1])
    raises("bytes", f2.fairy2i_pack, codes, packed=torch.zeros(16, dtype=torch.uint8))
    raises("GPU", f2.fairy2i_pack, codes)
    packed, scales = layer()
    raises("bytes", f2.fairy2i_dequantize, packed[:-16], scales, m)
    raises("shape", f2.fairy2i_dequantize, packed, scales[..., :1], m)
    raises("shape", f2.fairy2i_dequantize, packed, scales, m, R=torch.zeros((2 * n, 2 * m - 2)))
    raises("GPU", f2.fairy2i_dequantize, packed, scales, m)


def test_gemv_checks():
    packed, scales = layer()
    x = torch.zeros((B, 2 * m), dtype=torch.bfloat16)
    raises("dtype", f2.fairy2i_gemv, packed, scales, x.to(torch.float16))
    raises("shape", f2.fairy2i_gemv, packed, scales, x[:, :-1])
    raises("contiguous", f2.fairy2i_gemv, packed, scales, torch.zeros((2 * m, B), dtype=torch.bfloat16).t())
    raises("bytes", f2.fairy2i_gemv, packed[:-16], scales, x, y=torch.zeros((B, 2 * n)))
    raises("dtype", f2.fairy2i_gemv, packed, scales.double(), x)
    raises("shape", f2.fairy2i_gemv, packed, scales, x, y=torch.zeros((B, 2 * n - 2)))
    raises("dtype", f2.fairy2i_gemv, packed, scales, x, y=torch.zeros((B, 2 * n), dtype=torch.int32))
    raises("GPU", f2.fairy2i_gemv, packed, scales, x, y=torch.zeros((B, 2 * n)))


def test_digit_form_checks():
    x = torch.zeros((B, 2 * m), dtype=torch.bfloat16)
    raises("GPU", f2.fairy2i_x_digits, x)
    raises("GPU", f2.fairy2i_x_digits_f6, x)
    short = f2.XDigits(torch.zeros(16, dtype=torch.uint8), B, m, f2.X_DIGITS_F6)
    raises("bytes", f2.fairy2i_x_digits_f6, x, out=short)
    other = f2.XDigits(torch.zeros(f2.fairy2i_x_digits_f6_bytes(m, 1), dtype=torch.uint8), 1, m, f2.X_DIGITS_F6)
    raises("made for", f2.fairy2i_x_digits_f6, x, out=other)
    packed, scales = layer()
    raises("bytes", f2.fairy2i_gemv, packed, scales, short)


def test_grouped_and_strided_checks():
    packed, scales = layer()
    x = torch.zeros((B, 2 * m), dtype=torch.bfloat16)
    y = torch.zeros((B, 2 * n))
    raises("no items", f2.fairy2i_gemv_grouped, [])
    raises("bytes", f2.fairy2i_gemv_grouped, [(packed, scales, x, y), (packed[:-16], scales, x, y)])
    raises("shape", f2.fairy2i_gemv_grouped, [(packed, scales, x, y[:, :-2])])
    x2 = torch.zeros((B, 4 * m), dtype=torch.bfloat16)
    raises("m =", f2.fairy2i_gemv_grouped, [(packed, scales, x, y), (packed, scales, x2, y)])
    x1 = torch.zeros((1, 2 * m), dtype=torch.bfloat16)
    raises("B =", f2.fairy2i_gemv_grouped, [(packed, scales, x, y), (packed, scales, x1, y[:1])])
    raises("dtype", f2.fairy2i_gemv_grouped, [(packed, scales, x, y), (packed, scales, x, y.bfloat16())])
    s3 = torch.zeros((n, 3, 2, 2))
    raises("T =", f2.fairy2i_gemv_grouped, [(packed, scales, x, y), (torch.zeros(f2.fairy2i_packed_bytes(n, m, 3), dtype=torch.uint8), s3, x, y)])
    raises("GPU", f2.fairy2i_gemv_grouped, [(packed, scales, x, y)])
    pool = packed.unsqueeze(0).repeat(3, 1)
    ys = torch.zeros((3, B, 2 * n))
    raises("bytes per matrix", f2.fairy2i_gemv_strided, pool[:, :-16], scales, x, ys)
    raises("matrices", f2.fairy2i_gemv_strided, pool, scales.unsqueeze(0).repeat(2, 1, 1, 1, 1), x, ys)
    raises("shape", f2.fairy2i_gemv_strided, pool, scales, x, ys[:, :1])
    raises("contiguous", f2.fairy2i_gemv_strided, pool, scales, x, torch.zeros((3, 2 * n, B)).transpose(1, 2))
    raises("overlap", f2.fairy2i_gemv_strided, pool, scales, x, torch.zeros((1, B, 2 * n)).expand(3, -1, -1))
    raises("GPU", f2.fairy2i_gemv_strided, pool, scales, x, ys)
    raises("GPU", f2.fairy2i_gemv_strided, packed.unsqueeze(0).expand(3, -1), scales, x, ys)   # shared codes


def test_act_quant_and_gemm_checks():
    N = 5
    x = torch.zeros((N, 2 * m), dtype=torch.bfloat16)
    raises("shape", f2.fairy2i_act_quant, x, q=torch.zeros((N, 2 * m - 8), dtype=torch.int8))
    raises("dtype", f2.fairy2i_act_quant, x, delta=torch.zeros(N, dtype=torch.float64))
    raises("GPU", f2.fairy2i_act_quant, x)
    packed, scales = layer()
    raises("bytes", f2.fairy2i_gemm, packed[:-16], scales, x)
    q = torch.zeros((N, 2 * m), dtype=torch.int8)
    with pytest.raises(TypeError):
        f2.fairy2i_gemm(packed, scales, q)                              # int8 x needs its delta
    raises("shape", f2.fairy2i_gemm, packed, scales, q, x_scale=torch.zeros(N + 1))
    raises("shape", f2.fairy2i_gemm, packed, scales, x, y=torch.zeros((N, 2 * n), dtype=torch.int32))
    ws = torch.zeros(f2.fairy2i_gemm_workspace_bytes(n, m, T, N, f2.BF16), dtype=torch.uint8)
    raises("bytes", f2.fairy2i_gemm, packed, scales, x, workspace=ws[:-16])
    raises("GPU", f2.fairy2i_gemm, packed, scales, x, workspace=ws)
    raises("GPU", f2.fairy2i_gemm, packed, scales, q, x_scale=torch.zeros(N))


class _Recorder:
    """Stands in for the library: records each compute call's arguments (sizes and helpers go to
    the real library).  Lets the CPU run every binding function through to its C call."""

    def __init__(self, real):
        self.real, self.calls = real, []

    def __getattr__(self, name):
        fn = getattr(self.real, name)
        if name.endswith("_bytes") or name in ("fairy2i_last_error", "fairy2i_status_string"):
            return fn

        def record(*args):
            self.calls.append((name, args))
            return 0
        return record


@pytest.fixture
def recorder(monkeypatch):
    rec = _Recorder(f2.lib())
    monkeypatch.setattr(f2, "lib", lambda: rec)
    monkeypatch.setattr(f2, "_gpu", lambda *named: None)       # CPU tensors stand in for GPU ones
    monkeypatch.setattr(f2, "_stream", lambda stream=None: None)
    return rec


def test_marshalling_reaches_the_c_call(recorder):
    """Every binding function, given well-formed tensors, computes its C arguments (sizes, dtype
    codes, strides) without error; the recorded integer arguments are the documented ones."""
    R = torch.zeros((2 * n, 2 * m), dtype=torch.float32)
    f2.fairy2i_quantize(R, T, want_scales64=True, want_codes=True)
    f2.fairy2i_quantize(R.bfloat16(), T)
    f2.fairy2i_quantize_tensor(R, T)
    packed, scales = layer()
    f2.fairy2i_pack(torch.zeros((T, 2, n, m), dtype=torch.uint8))
    f2.fairy2i_dequantize(packed, scales, m, R_dtype=torch.bfloat16)
    x = torch.zeros((B, 2 * m), dtype=torch.bfloat16)
    xd = f2.fairy2i_x_digits_f6(x)
    f2.fairy2i_x_digits(x)
    f2.fairy2i_gemv(packed, scales, x)
    f2.fairy2i_gemv(packed, scales, xd, algo=f2.GEMV_MFMA_F4)
    f2.fairy2i_gemv_grouped([(packed, scales, x, torch.zeros((B, 2 * n)))] * 2)
    f2.fairy2i_gemv_strided(packed.unsqueeze(0).expand(3, -1), scales, x, torch.zeros((3, B, 2 * n)))
    f2.fairy2i_act_quant(x)
    f2.fairy2i_gemm(packed, scales, x)
    f2.fairy2i_gemm(packed, scales, x.float(), y_dtype=torch.int32)
    names = [c[0] for c in recorder.calls]
    assert names == ["fairy2i_quantize", "fairy2i_quantize_bf16", "fairy2i_quantize_tensor", "fairy2i_pack",
                     "fairy2i_dequantize", "fairy2i_x_digits_f6", "fairy2i_x_digits", "fairy2i_gemv",
                     "fairy2i_gemv", "fairy2i_gemv_grouped", "fairy2i_gemv_strided", "fairy2i_act_quant",
                     "fairy2i_gemm", "fairy2i_gemm"]
    args = dict((c[0] + str(k), c[1]) for k, c in enumerate(recorder.calls))
    assert args["fairy2i_quantize0"][1:4] == (2 * n, 2 * m, T)
    assert args["fairy2i_quantize_tensor2"][1:5] == (f2.F32, 2 * n, 2 * m, T)
    assert args["fairy2i_pack3"][1:4] == (n, m, T)
    assert args["fairy2i_dequantize4"][2:5] == (n, m, T) and args["fairy2i_dequantize4"][6] == f2.BF16
    assert args["fairy2i_gemv7"][2:5] == (n, m, T) and args["fairy2i_gemv7"][6:8] == (f2.BF16, B)
    assert args["fairy2i_gemv8"][6:8] == (f2.X_DIGITS_F6, B)
    assert args["fairy2i_gemv_grouped9"][1:6] == (2, m, T, f2.BF16, B)
    st = args["fairy2i_gemv_strided10"]
    assert st[1] == 0 and st[3] == 0 and st[4:7] == (n, m, T) and st[11] == 2 * n * B and st[13] == 3
    assert args["fairy2i_gemm13"][2:5] == (n, m, T) and args["fairy2i_gemm13"][10] == f2.I32
