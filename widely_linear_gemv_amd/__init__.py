"""Python binding of libfairy2i.so (the C ABI declared in include/fairy2i.h).

Argument marshalling only: every step of the hot path runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream.  The functions carry the C names
and take torch tensors; output tensors are allocated here when the caller passes none.

The library is built in-tree by `python -m widely_linear_gemv_amd.build`.  If it is missing,
every call raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfairy2i.so")

FAIRY2I_OK = 0
STATUS_NAMES = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_STAGES", 4: "ERR_DTYPE",
                5: "ERR_ALIGN", 6: "ERR_WORKSPACE", 7: "ERR_HIP"}
F32, BF16, I8, I32, X_DIGITS, X_DIGITS_F6 = 0, 1, 2, 3, 4, 5
GEMV_AUTO, GEMV_VALU, GEMV_MFMA, GEMV_MFMA_BF16, GEMV_MFMA_I8, GEMV_MFMA_F4 = 0, 1, 2, 3, 4, 5

_DTYPE = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.int32: I32}

# Every symbol include/fairy2i.h declares: name -> (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
SIGNATURES = {
    "fairy2i_quantize": (_INT, [_P, _I64, _I64, _INT, _P, _P, _P, _P, _P]),
    "fairy2i_quantize_bf16": (_INT, [_P, _I64, _I64, _INT, _P, _P, _P, _P, _P]),
    "fairy2i_quantize_tensor_workspace_bytes": (_SZ, [_I64, _I64, _INT]),
    "fairy2i_quantize_tensor": (_INT, [_P, _INT, _I64, _I64, _INT, _P, _SZ, _P, _P, _P, _P, _P]),
    "fairy2i_pack": (_INT, [_P, _I64, _I64, _INT, _P, _P]),
    "fairy2i_packed_bytes": (_SZ, [_I64, _I64, _INT]),
    "fairy2i_dequantize": (_INT, [_P, _P, _I64, _I64, _INT, _P, _INT, _P]),
    "fairy2i_x_digits_bytes": (_SZ, [_I64, _I64]),
    "fairy2i_x_digits": (_INT, [_P, _INT, _I64, _I64, _P, _P]),
    "fairy2i_x_digits_f6_bytes": (_SZ, [_I64, _I64]),
    "fairy2i_x_digits_f6": (_INT, [_P, _INT, _I64, _I64, _P, _P]),
    "fairy2i_gemv": (_INT, [_P, _P, _I64, _I64, _INT, _P, _INT, _I64, _P, _INT, _INT, _P]),
    "fairy2i_act_quant": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P]),
    "fairy2i_gemm_workspace_bytes": (_SZ, [_I64, _I64, _INT, _I64, _INT]),
    "fairy2i_gemm": (_INT, [_P, _P, _I64, _I64, _INT, _P, _INT, _P, _I64, _P, _INT, _P, _SZ, _P]),
    "fairy2i_status_string": (ctypes.c_char_p, [_INT]),
    "fairy2i_last_error": (ctypes.c_char_p, []),
    "fairy2i_abi_version": (_INT, []),
}



class GemvItem(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("n", ctypes.c_int64)]


SIGNATURES["fairy2i_gemv_grouped"] = (_INT, [ctypes.POINTER(GemvItem), _INT, _I64, _INT, _INT, _I64,
                                              _INT, _INT, _P])
SIGNATURES["fairy2i_gemv_strided"] = (_INT, [_P, _I64, _P, _I64, _I64, _I64, _INT, _P, _INT, _I64, _P, _I64,
                                              _INT, _I64, _INT, _P])

_lib = None


class Fairy2iError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m widely_linear_gemv_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != FAIRY2I_OK:
        msg = lib().fairy2i_last_error().decode(errors="replace")
        raise Fairy2iError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def fairy2i_abi_version() -> int:
    return lib().fairy2i_abi_version()


def fairy2i_status_string(status: int) -> str:
    return lib().fairy2i_status_string(status).decode()


def fairy2i_last_error() -> str:
    return lib().fairy2i_last_error().decode(errors="replace")


def fairy2i_packed_bytes(n: int, m: int, T: int) -> int:
    return int(lib().fairy2i_packed_bytes(n, m, T))


def fairy2i_quantize_tensor_workspace_bytes(n: int, m: int, T: int) -> int:
    return int(lib().fairy2i_quantize_tensor_workspace_bytes(n, m, T))


def fairy2i_quantize(R: torch.Tensor, T: int, *, want_scales64: bool = False,
                     want_codes: bool = False, packed=None, scales=None, stream=None):
    """R fp32 or bf16 [2n][2m] on the GPU -> dict(packed (flat uint8), scales[, scales64][, codes])."""
    two_n, two_m = R.shape
    n, m = two_n // 2, two_m // 2
    dev = R.device
    packed = packed if packed is not None else torch.empty((fairy2i_packed_bytes(n, m, T),), dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty((n, T, 2, 2), dtype=torch.float32, device=dev)
    s64 = torch.empty((n, T, 2, 2), dtype=torch.float64, device=dev) if want_scales64 else None
    codes = torch.empty((T, 2, n, m), dtype=torch.uint8, device=dev) if want_codes else None
    fn = lib().fairy2i_quantize_bf16 if R.dtype == torch.bfloat16 else lib().fairy2i_quantize
    _check(fn(_ptr(R), two_n, two_m, T, _ptr(packed), _ptr(scales), _ptr(s64), _ptr(codes), _stream(stream)))
    out = {"packed": packed, "scales": scales}
    if s64 is not None:
        out["scales64"] = s64
    if codes is not None:
        out["codes"] = codes
    return out


def fairy2i_quantize_tensor(R: torch.Tensor, T: int, *, want_scales64: bool = False,
                            want_codes: bool = False, workspace=None, packed=None, scales=None,
                            stream=None):
    """fairy2i_quantize with per-tensor axis scales (every row of scales holds the same pairs)."""
    two_n, two_m = R.shape
    n, m = two_n // 2, two_m // 2
    dev = R.device
    if workspace is None:
        workspace = torch.empty((fairy2i_quantize_tensor_workspace_bytes(n, m, T),), dtype=torch.uint8, device=dev)
    packed = packed if packed is not None else torch.empty((fairy2i_packed_bytes(n, m, T),), dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty((n, T, 2, 2), dtype=torch.float32, device=dev)
    s64 = torch.empty((n, T, 2, 2), dtype=torch.float64, device=dev) if want_scales64 else None
    codes = torch.empty((T, 2, n, m), dtype=torch.uint8, device=dev) if want_codes else None
    _check(lib().fairy2i_quantize_tensor(_ptr(R), _DTYPE[R.dtype], two_n, two_m, T, _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(packed),
                                         _ptr(scales), _ptr(s64), _ptr(codes), _stream(stream)))
    out = {"packed": packed, "scales": scales}
    if s64 is not None:
        out["scales64"] = s64
    if codes is not None:
        out["codes"] = codes
    return out


def fairy2i_pack(codes: torch.Tensor, packed=None, stream=None) -> torch.Tensor:
    """codes uint8 [T][2][n][m] -> the packed form (flat uint8, fairy2i_packed_bytes)."""
    T, _, n, m = codes.shape
    packed = packed if packed is not None else torch.empty((fairy2i_packed_bytes(n, m, T),), dtype=torch.uint8, device=codes.device)
    _check(lib().fairy2i_pack(_ptr(codes), n, m, T, _ptr(packed), _stream(stream)))
    return packed


def fairy2i_dequantize(packed: torch.Tensor, scales: torch.Tensor, m: int, *, R_dtype=torch.float32,
                       R=None, stream=None) -> torch.Tensor:
    """packed form + scales [n][T][2][2] -> the real layer R^ [2n][2m] (fp32 or bf16)."""
    n, T = scales.shape[0], scales.shape[1]
    if R is None:
        R = torch.empty((2 * n, 2 * m), dtype=R_dtype, device=packed.device)
    _check(lib().fairy2i_dequantize(_ptr(packed), _ptr(scales), n, m, T, _ptr(R), _DTYPE[R.dtype],
                                    _stream(stream)))
    return R


class XDigits:
    """A digit form of decode-GEMV activations: the uint8 buffer, the B and m it was made with,
    and its dtype code (X_DIGITS: int8 digits of fairy2i_x_digits; X_DIGITS_F6: fp6 digits of
    fairy2i_x_digits_f6)."""

    def __init__(self, buf: torch.Tensor, B: int, m: int, dtype: int = X_DIGITS):
        self.buf, self.B, self.m, self.dtype = buf, B, m, dtype

    @property
    def device(self):
        return self.buf.device


def _x_cols(x) -> int:
    """Complex columns m of a GEMV/GEMM activation argument."""
    return x.m if isinstance(x, XDigits) else x.shape[1] // 2


def _x_args(x):
    """(pointer, x_dtype, B) of a GEMV activation argument: a [B][2m] tensor or an XDigits."""
    if isinstance(x, XDigits):
        return _ptr(x.buf), x.dtype, x.B
    return _ptr(x), _DTYPE[x.dtype], x.shape[0]


def fairy2i_x_digits_bytes(m: int, B: int) -> int:
    return int(lib().fairy2i_x_digits_bytes(m, B))


def fairy2i_x_digits(x: torch.Tensor, out: XDigits | None = None, stream=None) -> XDigits:
    """x [B][2m] (bf16 / fp32, B <= 2) -> its exact int8 digit form for the int8 MFMA GEMV."""
    B, two_m = x.shape
    m = two_m // 2
    if out is None:
        out = XDigits(torch.empty((fairy2i_x_digits_bytes(m, B),), dtype=torch.uint8, device=x.device), B, m)
    _check(lib().fairy2i_x_digits(_ptr(x), _DTYPE[x.dtype], m, B, _ptr(out.buf), _stream(stream)))
    return out


def fairy2i_x_digits_f6_bytes(m: int, B: int) -> int:
    return int(lib().fairy2i_x_digits_f6_bytes(m, B))


def fairy2i_x_digits_f6(x: torch.Tensor, out: XDigits | None = None, stream=None) -> XDigits:
    """x [B][2m] (bf16 / fp32, B <= 2) -> its exact fp6 digit form for the fp4 MFMA GEMV."""
    B, two_m = x.shape
    m = two_m // 2
    if out is None:
        out = XDigits(torch.empty((fairy2i_x_digits_f6_bytes(m, B),), dtype=torch.uint8, device=x.device),
                      B, m, X_DIGITS_F6)
    _check(lib().fairy2i_x_digits_f6(_ptr(x), _DTYPE[x.dtype], m, B, _ptr(out.buf), _stream(stream)))
    return out


def fairy2i_gemv(packed: torch.Tensor, scales: torch.Tensor, x, *,
                 y_dtype=torch.float32, algo: int = GEMV_AUTO, y=None, stream=None) -> torch.Tensor:
    """packed form, scales [n][T][2][2], x [B][2m] (or its XDigits) -> y [B][2n].  n and T come
    from the scales, m from x."""
    n, T = scales.shape[0], scales.shape[1]
    m = _x_cols(x)
    xp, xdt, B = _x_args(x)
    if y is None:
        y = torch.empty((B, 2 * n), dtype=y_dtype, device=x.device)
    _check(lib().fairy2i_gemv(_ptr(packed), _ptr(scales), n, m, T, xp, xdt, B,
                              _ptr(y), _DTYPE[y.dtype], algo, _stream(stream)))
    return y


def fairy2i_gemv_grouped(items, *, algo: int = GEMV_AUTO, stream=None):
    """items: sequence of (packed, scales, x, y) tensor tuples sharing m, T, B and dtypes; each y
    [B][2n] is preallocated by the caller.  Returns the list of y."""
    items = list(items)
    arr = (GemvItem * len(items))()
    for k, (packed, scales, x, y) in enumerate(items):
        arr[k] = GemvItem(packed.data_ptr(), scales.data_ptr(), _x_args(x)[0], y.data_ptr(), scales.shape[0])
    _, scales0, x0, y0 = items[0]
    T = scales0.shape[1]
    _, xdt, B = _x_args(x0)
    _check(lib().fairy2i_gemv_grouped(arr, len(items), _x_cols(x0), T, xdt, B,
                                      _DTYPE[y0.dtype], algo, _stream(stream)))
    return [it[3] for it in items]


def fairy2i_gemv_strided(packed: torch.Tensor, scales: torch.Tensor, x, y: torch.Tensor, *,
                         algo: int = GEMV_AUTO, stream=None):
    """A strided batch of GEMVs sharing x: packed [batch][bytes] uint8, scales [batch][n][T][2][2]
    (or [n][T][2][2], shared by all), y [batch][B][2n] preallocated; the strides are those of the
    tensors' first dimension (each matrix's slice contiguous).  Returns y."""
    if packed.dim() != 2 or y.dim() != 3 or scales.dim() not in (4, 5):
        raise ValueError("fairy2i_gemv_strided: packed [batch][bytes], scales [batch][n][T][2][2] or "
                         "[n][T][2][2], y [batch][B][2n]")
    batch = packed.shape[0]
    n, T = scales.shape[-4], scales.shape[-3]
    s_stride = scales.stride(0) if scales.dim() == 5 else 0
    xp, xdt, B = _x_args(x)
    _check(lib().fairy2i_gemv_strided(_ptr(packed), packed.stride(0), _ptr(scales), s_stride, n,
                                      _x_cols(x), T, xp, xdt, B, _ptr(y), y.stride(0), _DTYPE[y.dtype],
                                      batch, algo, _stream(stream)))
    return y


def fairy2i_act_quant(x: torch.Tensor, q=None, delta=None, stream=None):
    """x [N][2m] (fp32 / bf16) -> (q int8 [N][2m], delta fp32 [N])."""
    N, two_m = x.shape
    q = q if q is not None else torch.empty((N, two_m), dtype=torch.int8, device=x.device)
    delta = delta if delta is not None else torch.empty((N,), dtype=torch.float32, device=x.device)
    _check(lib().fairy2i_act_quant(_ptr(x), _DTYPE[x.dtype], N, two_m, _ptr(q), _ptr(delta), _stream(stream)))
    return q, delta


def fairy2i_gemm_workspace_bytes(n: int, m: int, T: int, N: int, x_dtype: int) -> int:
    return int(lib().fairy2i_gemm_workspace_bytes(n, m, T, N, x_dtype))


def fairy2i_gemm(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, *,
                 x_scale=None, y_dtype=torch.float32, y=None, workspace=None, stream=None):
    """Prefill over N tokens.  x [N][2m] bf16/fp32 (x_scale receives delta if given) or int8
    (x_scale = delta input).  y_dtype float32/bfloat16 -> y [N][2n]; int32 -> raw
    accumulators [T][2][2][2][N][n]."""
    n, T = scales.shape[0], scales.shape[1]
    m = x.shape[1] // 2
    N = x.shape[0]
    if y is None:
        shape = (T, 2, 2, 2, N, n) if y_dtype == torch.int32 else (N, 2 * n)
        y = torch.empty(shape, dtype=y_dtype, device=x.device)
    if workspace is None:
        nbytes = fairy2i_gemm_workspace_bytes(n, m, T, N, _DTYPE[x.dtype])
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib().fairy2i_gemm(_ptr(packed), _ptr(scales), n, m, T, _ptr(x), _DTYPE[x.dtype],
                              _ptr(x_scale), N, _ptr(y), _DTYPE[y.dtype], _ptr(workspace), ws_bytes,
                              _stream(stream)))
    return y
