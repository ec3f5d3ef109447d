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
# FAIRY2I_LIB selects another build of the same library (the host-sanitized one, for instance).
LIB_PATH = os.environ.get("FAIRY2I_LIB") or os.path.join(_HERE, "libfairy2i.so")

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
    "fairy2i_gemm_noalloc_max_bytes": (_SZ, []),
    "fairy2i_gemm_noalloc": (_INT, [_P, _P, _I64, _I64, _INT, _P, _INT, _P, _I64, _P, _INT, _P]),
    "fairy2i_status_string": (ctypes.c_char_p, [_INT]),
    "fairy2i_last_error": (ctypes.c_char_p, []),
    "fairy2i_abi_version": (_INT, []),
}



class GemvItem(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("n", ctypes.c_int64)]


SIGNATURES["fairy2i_quantize_grouped"] = (_INT, [_INT, ctypes.POINTER(ctypes.c_void_p), _INT, _I64, _I64, _INT,
                                                  ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                                  ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                                  _P])
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


# ---- argument checks --------------------------------------------------------------------
# The C ABI takes bare device pointers and no buffer sizes: its kernels size every access from the
# call's n, m, T and B.  So before a pointer is passed on, each tensor is checked here for being a
# contiguous GPU tensor of the right dtype, shape and size; a mismatch raises ValueError and nothing
# is launched.  (Checks run dtype -> shape -> size -> layout -> device, so a CPU tensor that is
# otherwise right fails on the device check.)

def _tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    return t


def _dtype(t, name, *allowed):
    if t.dtype not in allowed:
        raise ValueError(f"{name}: dtype {t.dtype}, need one of {', '.join(str(a) for a in allowed)}")


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, need {tuple(shape)}")


def _min_bytes(t, name, nbytes):
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, need at least {nbytes}")


def _on_gpu(t, name, dev=None, contiguous=True):
    """Layout now; the device check is left to _gpu, after every other check of the call."""
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _gpu(*named):
    """(tensor, name) pairs: all on one GPU.  The last check before a call enters the library."""
    dev = None
    for t, name in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name}: must be on the GPU (got {t.device})")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name}: on {t.device}, the other operands are on {dev}")
        dev = t.device


def _scales_nT(scales, name="scales"):
    """(n, T) of an fp32 scales tensor [n][T][2][2]."""
    _tensor(scales, name)
    _dtype(scales, name, torch.float32)
    if scales.dim() != 4 or tuple(scales.shape[2:]) != (2, 2):
        raise ValueError(f"{name}: shape {tuple(scales.shape)}, need [n][T][2][2]")
    return scales.shape[0], scales.shape[1]


def _check_x(x, name="x", dtypes=(torch.float32, torch.bfloat16)):
    """Checks a GEMV activation argument (a [B][2m] tensor or an XDigits) up to its device."""
    if isinstance(x, XDigits):
        _tensor(x.buf, name + ".buf")
        _dtype(x.buf, name + ".buf", torch.uint8)
        nbytes = (fairy2i_x_digits_f6_bytes if x.dtype == X_DIGITS_F6 else fairy2i_x_digits_bytes)(x.m, x.B)
        _min_bytes(x.buf, name + ".buf", nbytes)
        _on_gpu(x.buf, name + ".buf")
        return x.buf.device
    _tensor(x, name)
    _dtype(x, name, *dtypes)
    if x.dim() != 2 or x.shape[1] % 2:
        raise ValueError(f"{name}: shape {tuple(x.shape)}, need [B][2m]")
    _on_gpu(x, name)
    return x.device


def _check_layer(packed, scales, m, dev, pname="packed", sname="scales"):
    """packed bytes and scales of an n x m layer, on device dev; returns (n, T)."""
    n, T = _scales_nT(scales, sname)
    _tensor(packed, pname)
    _dtype(packed, pname, torch.uint8)
    _min_bytes(packed, pname, fairy2i_packed_bytes(n, m, T))
    _on_gpu(packed, pname, dev)
    _on_gpu(scales, sname, dev)
    return n, T


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


def _check_weight(R, name="R"):
    _tensor(R, name)
    _dtype(R, name, torch.float32, torch.bfloat16)
    if R.dim() != 2 or R.shape[0] % 2 or R.shape[1] % 2:
        raise ValueError(f"{name}: shape {tuple(R.shape)}, need [2n][2m]")
    _on_gpu(R, name)
    return R.shape[0] // 2, R.shape[1] // 2, R.device


def _quant_outputs(packed, scales, n, m, T, dev):
    """The quantizers' packed and scales outputs: allocated when None, checked otherwise."""
    if packed is None:
        packed = torch.empty((fairy2i_packed_bytes(n, m, T),), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((n, T, 2, 2), dtype=torch.float32, device=dev)
    _tensor(scales, "scales")
    _dtype(scales, "scales", torch.float32)
    _shape(scales, "scales", (n, T, 2, 2))
    _check_layer(packed, scales, m, dev)
    return packed, scales


def fairy2i_quantize(R: torch.Tensor, T: int, *, want_scales64: bool = False,
                     want_codes: bool = False, packed=None, scales=None, stream=None):
    """R fp32 or bf16 [2n][2m] on the GPU -> dict(packed (flat uint8), scales[, scales64][, codes])."""
    n, m, dev = _check_weight(R)
    packed, scales = _quant_outputs(packed, scales, n, m, T, dev)
    s64 = torch.empty((n, T, 2, 2), dtype=torch.float64, device=dev) if want_scales64 else None
    codes = torch.empty((T, 2, n, m), dtype=torch.uint8, device=dev) if want_codes else None
    fn = lib().fairy2i_quantize_bf16 if R.dtype == torch.bfloat16 else lib().fairy2i_quantize
    _gpu((R, "R"), (packed, "packed"), (scales, "scales"), (s64, "scales64"), (codes, "codes"))
    _check(fn(_ptr(R), 2 * n, 2 * m, T, _ptr(packed), _ptr(scales), _ptr(s64), _ptr(codes), _stream(stream)))
    out = {"packed": packed, "scales": scales}
    if s64 is not None:
        out["scales64"] = s64
    if codes is not None:
        out["codes"] = codes
    return out


def fairy2i_quantize_grouped(Rs, T: int, *, want_scales64: bool = False, want_codes: bool = False,
                             packed=None, scales=None, stream=None):
    """fairy2i_quantize on a list of layers of one shape and dtype (fp32 or bf16 [2n][2m] on one
    GPU), in shared launches; each layer's result equals its own fairy2i_quantize call.  packed and
    scales: None (allocated) or lists of one output per layer.  Returns a list of dicts like
    fairy2i_quantize."""
    Rs = list(Rs)
    if not Rs:
        return []
    n, m, dev = _check_weight(Rs[0], "R[0]")
    for k, R in enumerate(Rs):
        nk, mk, _ = _check_weight(R, f"R[{k}]")
        if (nk, mk) != (n, m) or R.dtype != Rs[0].dtype:
            raise ValueError(f"R[{k}]: {R.dtype} [{2 * nk}][{2 * mk}], the group is {Rs[0].dtype} [{2 * n}][{2 * m}]")
    count = len(Rs)
    for name, given in (("packed", packed), ("scales", scales)):
        if given is not None and len(given) != count:
            raise ValueError(f"{name}: {len(given)} outputs for {count} layers")
    outs = [_quant_outputs(None if packed is None else packed[k], None if scales is None else scales[k], n, m, T, dev)
            for k in range(count)]
    s64 = [torch.empty((n, T, 2, 2), dtype=torch.float64, device=dev) for _ in range(count)] if want_scales64 else None
    codes = [torch.empty((T, 2, n, m), dtype=torch.uint8, device=dev) for _ in range(count)] if want_codes else None
    named = [(R, f"R[{k}]") for k, R in enumerate(Rs)]
    named += [(t, f"{name}[{k}]") for k, (pk, sc) in enumerate(outs) for t, name in ((pk, "packed"), (sc, "scales"))]
    named += [(t, f"scales64[{k}]") for k, t in enumerate(s64 or [])] + [(t, f"codes[{k}]") for k, t in enumerate(codes or [])]
    _gpu(*named)
    arr = lambda ts: (ctypes.c_void_p * count)(*[t.data_ptr() for t in ts])
    _check(lib().fairy2i_quantize_grouped(count, arr(Rs), _DTYPE[Rs[0].dtype], 2 * n, 2 * m, T,
                                          arr([o[0] for o in outs]), arr([o[1] for o in outs]),
                                          arr(s64) if s64 else None, arr(codes) if codes else None, _stream(stream)))
    res = []
    for k, (pk, sc) in enumerate(outs):
        d = {"packed": pk, "scales": sc}
        if s64:
            d["scales64"] = s64[k]
        if codes:
            d["codes"] = codes[k]
        res.append(d)
    return res


def fairy2i_quantize_tensor(R: torch.Tensor, T: int, *, want_scales64: bool = False,
                            want_codes: bool = False, workspace=None, packed=None, scales=None,
                            stream=None):
    """fairy2i_quantize with per-tensor axis scales (every row of scales holds the same pairs)."""
    n, m, dev = _check_weight(R)
    two_n, two_m = 2 * n, 2 * m
    if workspace is None:
        workspace = torch.empty((fairy2i_quantize_tensor_workspace_bytes(n, m, T),), dtype=torch.uint8, device=dev)
    _tensor(workspace, "workspace")
    _min_bytes(workspace, "workspace", fairy2i_quantize_tensor_workspace_bytes(n, m, T))
    _on_gpu(workspace, "workspace", dev)
    packed, scales = _quant_outputs(packed, scales, n, m, T, dev)
    s64 = torch.empty((n, T, 2, 2), dtype=torch.float64, device=dev) if want_scales64 else None
    codes = torch.empty((T, 2, n, m), dtype=torch.uint8, device=dev) if want_codes else None
    _gpu((R, "R"), (workspace, "workspace"), (packed, "packed"), (scales, "scales"), (s64, "scales64"),
         (codes, "codes"))
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
    _tensor(codes, "codes")
    _dtype(codes, "codes", torch.uint8)
    if codes.dim() != 4 or codes.shape[1] != 2:
        raise ValueError(f"codes: shape {tuple(codes.shape)}, need [T][2][n][m]")
    _on_gpu(codes, "codes")
    T, _, n, m = codes.shape
    packed = packed if packed is not None else torch.empty((fairy2i_packed_bytes(n, m, T),), dtype=torch.uint8, device=codes.device)
    _tensor(packed, "packed")
    _dtype(packed, "packed", torch.uint8)
    _min_bytes(packed, "packed", fairy2i_packed_bytes(n, m, T))
    _on_gpu(packed, "packed", codes.device)
    _gpu((codes, "codes"), (packed, "packed"))
    _check(lib().fairy2i_pack(_ptr(codes), n, m, T, _ptr(packed), _stream(stream)))
    return packed


def fairy2i_dequantize(packed: torch.Tensor, scales: torch.Tensor, m: int, *, R_dtype=torch.float32,
                       R=None, stream=None) -> torch.Tensor:
    """packed form + scales [n][T][2][2] -> the real layer R^ [2n][2m] (fp32 or bf16)."""
    _tensor(packed, "packed")
    n, T = _check_layer(packed, scales, m, packed.device)
    if R is None:
        R = torch.empty((2 * n, 2 * m), dtype=R_dtype, device=packed.device)
    _tensor(R, "R")
    _dtype(R, "R", torch.float32, torch.bfloat16)
    _shape(R, "R", (2 * n, 2 * m))
    _on_gpu(R, "R", packed.device)
    _gpu((packed, "packed"), (scales, "scales"), (R, "R"))
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


def _x_tensor(x):
    """The device tensor of a GEMV activation argument."""
    return x.buf if isinstance(x, XDigits) else x


def _x_cols(x) -> int:
    """Complex columns m of a GEMV/GEMM activation argument."""
    return x.m if isinstance(x, XDigits) else x.shape[1] // 2


def _x_args(x):
    """(pointer, x_dtype, B) of a GEMV activation argument: a [B][2m] tensor or an XDigits."""
    if isinstance(x, XDigits):
        return _ptr(x.buf), x.dtype, x.B
    return _ptr(x), _DTYPE[x.dtype], x.shape[0]


def _check_digits_out(out, B, m, dtype, dev):
    if not isinstance(out, XDigits):
        raise TypeError("out: expected an XDigits")
    if out.B != B or out.m != m or out.dtype != dtype:
        raise ValueError(f"out: made for B={out.B}, m={out.m}, dtype {out.dtype}; this x needs B={B}, m={m}, "
                         f"dtype {dtype}")
    _check_x(out, "out")
    if out.buf.device != dev:
        raise ValueError(f"out: on {out.buf.device}, x is on {dev}")


def fairy2i_x_digits_bytes(m: int, B: int) -> int:
    return int(lib().fairy2i_x_digits_bytes(m, B))


def fairy2i_x_digits(x: torch.Tensor, out: XDigits | None = None, stream=None) -> XDigits:
    """x [B][2m] (bf16 / fp32, B <= 2) -> its exact int8 digit form for the int8 MFMA GEMV."""
    _check_x(x)
    B, two_m = x.shape
    m = two_m // 2
    if out is None:
        out = XDigits(torch.empty((fairy2i_x_digits_bytes(m, B),), dtype=torch.uint8, device=x.device), B, m)
    _check_digits_out(out, B, m, X_DIGITS, x.device)
    _gpu((x, "x"), (out.buf, "out"))
    _check(lib().fairy2i_x_digits(_ptr(x), _DTYPE[x.dtype], m, B, _ptr(out.buf), _stream(stream)))
    return out


def fairy2i_x_digits_f6_bytes(m: int, B: int) -> int:
    return int(lib().fairy2i_x_digits_f6_bytes(m, B))


def fairy2i_x_digits_f6(x: torch.Tensor, out: XDigits | None = None, stream=None) -> XDigits:
    """x [B][2m] (bf16 / fp32, B <= 2) -> its exact fp6 digit form for the fp4 MFMA GEMV."""
    _check_x(x)
    B, two_m = x.shape
    m = two_m // 2
    if out is None:
        out = XDigits(torch.empty((fairy2i_x_digits_f6_bytes(m, B),), dtype=torch.uint8, device=x.device),
                      B, m, X_DIGITS_F6)
    _check_digits_out(out, B, m, X_DIGITS_F6, x.device)
    _gpu((x, "x"), (out.buf, "out"))
    _check(lib().fairy2i_x_digits_f6(_ptr(x), _DTYPE[x.dtype], m, B, _ptr(out.buf), _stream(stream)))
    return out


def _check_y(y, shape, dev, name="y"):
    _tensor(y, name)
    _dtype(y, name, torch.float32, torch.bfloat16)
    _shape(y, name, shape)
    _on_gpu(y, name, dev)


def fairy2i_gemv(packed: torch.Tensor, scales: torch.Tensor, x, *,
                 y_dtype=torch.float32, algo: int = GEMV_AUTO, y=None, stream=None) -> torch.Tensor:
    """packed form, scales [n][T][2][2], x [B][2m] (or its XDigits) -> y [B][2n].  n and T come
    from the scales, m from x."""
    dev = _check_x(x)
    m = _x_cols(x)
    n, T = _check_layer(packed, scales, m, dev)
    xp, xdt, B = _x_args(x)
    if y is None:
        y = torch.empty((B, 2 * n), dtype=y_dtype, device=dev)
    _check_y(y, (B, 2 * n), dev)
    _gpu((packed, "packed"), (scales, "scales"), (_x_tensor(x), "x"), (y, "y"))
    _check(lib().fairy2i_gemv(_ptr(packed), _ptr(scales), n, m, T, xp, xdt, B,
                              _ptr(y), _DTYPE[y.dtype], algo, _stream(stream)))
    return y


def fairy2i_gemv_grouped(items, *, algo: int = GEMV_AUTO, stream=None):
    """items: sequence of (packed, scales, x, y) tensor tuples sharing m, T, B and dtypes; each y
    [B][2n] is preallocated by the caller.  Returns the list of y."""
    items = list(items)
    if not items:
        raise ValueError("fairy2i_gemv_grouped: no items")
    arr = (GemvItem * len(items))()
    _, scales0, x0, y0 = items[0]
    dev = _check_x(x0, "items[0].x")
    m0 = _x_cols(x0)
    _, xdt0, B0 = _x_args(x0)
    T0 = _scales_nT(scales0, "items[0].scales")[1]
    _tensor(y0, "items[0].y")
    for k, (packed, scales, x, y) in enumerate(items):
        if _check_x(x, f"items[{k}].x") != dev:
            raise ValueError(f"items[{k}]: on another device than items[0]")
        if _x_cols(x) != m0 or _x_args(x)[1:] != (xdt0, B0):
            raise ValueError(f"items[{k}]: x has m = {_x_cols(x)}, dtype {_x_args(x)[1]}, B = {_x_args(x)[2]}; "
                             f"items[0] has m = {m0}, dtype {xdt0}, B = {B0}")
        n, T = _check_layer(packed, scales, m0, dev, f"items[{k}].packed", f"items[{k}].scales")
        if T != T0:
            raise ValueError(f"items[{k}]: T = {T}, items[0] has T = {T0}")
        _check_y(y, (B0, 2 * n), dev, f"items[{k}].y")
        if y.dtype != y0.dtype:
            raise ValueError(f"items[{k}].y: dtype {y.dtype}, items[0].y has {y0.dtype}")
        arr[k] = GemvItem(packed.data_ptr(), scales.data_ptr(), _x_args(x)[0], y.data_ptr(), n)
    T = scales0.shape[1]
    _, xdt, B = _x_args(x0)
    _gpu(*[(t, f"items[{k}]") for k, it in enumerate(items) for t in (it[0], it[1], _x_tensor(it[2]), it[3])])
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
    dev = _check_x(x)
    m = _x_cols(x)
    xp, xdt, B = _x_args(x)
    n, T = _scales_nT(scales[0] if scales.dim() == 5 else scales)
    _dtype(packed, "packed", torch.uint8)
    if packed.shape[1] < fairy2i_packed_bytes(n, m, T):
        raise ValueError(f"packed: {packed.shape[1]} bytes per matrix, need at least {fairy2i_packed_bytes(n, m, T)}")
    if scales.dim() == 5 and scales.shape[0] != batch:
        raise ValueError(f"scales: {scales.shape[0]} matrices, packed has {batch}")
    _dtype(y, "y", torch.float32, torch.bfloat16)
    if tuple(y.shape) != (batch, B, 2 * n):
        raise ValueError(f"y: shape {tuple(y.shape)}, need {(batch, B, 2 * n)}")
    # each matrix's slice must be contiguous; the first dimension may have any stride >= 0
    if packed.stride(1) != 1 or not y[0].is_contiguous() or not (scales[0] if scales.dim() == 5 else scales).is_contiguous():
        raise ValueError("fairy2i_gemv_strided: each matrix's packed bytes, scales and outputs must be contiguous")
    if batch > 1 and y.stride(0) < y[0].numel():
        raise ValueError("y: the outputs of different matrices overlap")
    for t, name in ((packed, "packed"), (scales, "scales"), (y, "y")):
        _on_gpu(t, name, dev, contiguous=False)
    s_stride = scales.stride(0) if scales.dim() == 5 else 0
    _gpu((packed, "packed"), (scales, "scales"), (_x_tensor(x), "x"), (y, "y"))
    _check(lib().fairy2i_gemv_strided(_ptr(packed), packed.stride(0), _ptr(scales), s_stride, n,
                                      _x_cols(x), T, xp, xdt, B, _ptr(y), y.stride(0), _DTYPE[y.dtype],
                                      batch, algo, _stream(stream)))
    return y


def fairy2i_act_quant(x: torch.Tensor, q=None, delta=None, stream=None):
    """x [N][2m] (fp32 / bf16) -> (q int8 [N][2m], delta fp32 [N])."""
    dev = _check_x(x)
    N, two_m = x.shape
    q = q if q is not None else torch.empty((N, two_m), dtype=torch.int8, device=dev)
    delta = delta if delta is not None else torch.empty((N,), dtype=torch.float32, device=dev)
    _tensor(q, "q")
    _dtype(q, "q", torch.int8)
    _shape(q, "q", (N, two_m))
    _on_gpu(q, "q", dev)
    _tensor(delta, "delta")
    _dtype(delta, "delta", torch.float32)
    _shape(delta, "delta", (N,))
    _on_gpu(delta, "delta", dev)
    _gpu((x, "x"), (q, "q"), (delta, "delta"))
    _check(lib().fairy2i_act_quant(_ptr(x), _DTYPE[x.dtype], N, two_m, _ptr(q), _ptr(delta), _stream(stream)))
    return q, delta


def fairy2i_gemm_workspace_bytes(n: int, m: int, T: int, N: int, x_dtype: int) -> int:
    return int(lib().fairy2i_gemm_workspace_bytes(n, m, T, N, x_dtype))


def fairy2i_gemm(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, *,
                 x_scale=None, y_dtype=torch.float32, y=None, workspace=None, stream=None):
    """Prefill over N tokens.  x [N][2m] bf16/fp32 (x_scale receives delta if given) or int8
    (x_scale = delta input).  y_dtype float32/bfloat16 -> y [N][2n]; int32 -> raw
    accumulators [T][2][2][2][N][n]."""
    dev = _check_x(x, dtypes=(torch.float32, torch.bfloat16, torch.int8))
    m = x.shape[1] // 2
    N = x.shape[0]
    n, T = _check_layer(packed, scales, m, dev)
    if x_scale is not None or x.dtype == torch.int8:
        _tensor(x_scale, "x_scale")
        _dtype(x_scale, "x_scale", torch.float32)
        _shape(x_scale, "x_scale", (N,))
        _on_gpu(x_scale, "x_scale", dev)
    if y is None:
        shape = (T, 2, 2, 2, N, n) if y_dtype == torch.int32 else (N, 2 * n)
        y = torch.empty(shape, dtype=y_dtype, device=dev)
    _tensor(y, "y")
    _dtype(y, "y", torch.float32, torch.bfloat16, torch.int32)
    _shape(y, "y", (T, 2, 2, 2, N, n) if y.dtype == torch.int32 else (N, 2 * n))
    _on_gpu(y, "y", dev)
    nbytes = fairy2i_gemm_workspace_bytes(n, m, T, N, _DTYPE[x.dtype])
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _tensor(workspace, "workspace")
        _min_bytes(workspace, "workspace", nbytes)
        _on_gpu(workspace, "workspace", dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _gpu((packed, "packed"), (scales, "scales"), (x, "x"), (x_scale, "x_scale"), (y, "y"), (workspace, "workspace"))
    _check(lib().fairy2i_gemm(_ptr(packed), _ptr(scales), n, m, T, _ptr(x), _DTYPE[x.dtype],
                              _ptr(x_scale), N, _ptr(y), _DTYPE[y.dtype], _ptr(workspace), ws_bytes,
                              _stream(stream)))
    return y


def fairy2i_gemm_noalloc_max_bytes() -> int:
    return int(lib().fairy2i_gemm_noalloc_max_bytes())


def fairy2i_gemm_noalloc(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, *,
                         x_scale=None, y: torch.Tensor, stream=None):
    """fairy2i_gemm without a workspace: the activation staging lives in the library's static
    device array (calls on one GPU must not overlap).  y is preallocated by the caller (no
    allocation at all here): float32/bfloat16 [N][2n], or int32 [T][2][2][2][N][n]."""
    dev = _check_x(x, dtypes=(torch.float32, torch.bfloat16, torch.int8))
    m = x.shape[1] // 2
    N = x.shape[0]
    n, T = _check_layer(packed, scales, m, dev)
    if x_scale is not None or x.dtype == torch.int8:
        _tensor(x_scale, "x_scale")
        _dtype(x_scale, "x_scale", torch.float32)
        _shape(x_scale, "x_scale", (N,))
        _on_gpu(x_scale, "x_scale", dev)
    _tensor(y, "y")
    _dtype(y, "y", torch.float32, torch.bfloat16, torch.int32)
    _shape(y, "y", (T, 2, 2, 2, N, n) if y.dtype == torch.int32 else (N, 2 * n))
    _on_gpu(y, "y", dev)
    _gpu((packed, "packed"), (scales, "scales"), (x, "x"), (x_scale, "x_scale"), (y, "y"))
    _check(lib().fairy2i_gemm_noalloc(_ptr(packed), _ptr(scales), n, m, T, _ptr(x), _DTYPE[x.dtype],
                                      _ptr(x_scale), N, _ptr(y), _DTYPE[y.dtype], _stream(stream)))
    return y

