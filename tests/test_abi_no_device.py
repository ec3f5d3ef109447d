"""Every compute entry point of the C ABI, called with valid arguments in a process that sees no
GPU (HIP_VISIBLE_DEVICES empty), returns FAIRY2I_ERR_HIP with the runtime's message -- no abort,
no crash.  The calls run in a child process, which first confirms that no device is visible and
otherwise makes no call at all (the pointers are placeholders, never dereferenced)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import ctypes, json, sys
sys.path.insert(0, ROOT)
import torch
if torch.cuda.device_count() != 0:
    print(json.dumps({"skipped": "a device is visible"}))
    sys.exit(0)
import widely_linear_gemv_amd as f2
L = f2.lib()
P = 1 << 20                       # 16-byte aligned placeholder address
S = None
n, m, T, B, N = 32, 64, 2, 1, 4
ws = L.fairy2i_quantize_tensor_workspace_bytes(n, m, T)
gws = L.fairy2i_gemm_workspace_bytes(n, m, T, N, f2.BF16)
items = (f2.GemvItem * 1)(f2.GemvItem(P, P, P, P, n))
calls = {
    "fairy2i_quantize": lambda: L.fairy2i_quantize(P, 2 * n, 2 * m, T, P, P, None, None, S),
    "fairy2i_quantize_bf16": lambda: L.fairy2i_quantize_bf16(P, 2 * n, 2 * m, T, P, P, None, None, S),
    "fairy2i_quantize_tensor": lambda: L.fairy2i_quantize_tensor(P, f2.F32, 2 * n, 2 * m, T, P, ws, P, P, None, None, S),
    "fairy2i_pack": lambda: L.fairy2i_pack(P, n, m, T, P, S),
    "fairy2i_dequantize": lambda: L.fairy2i_dequantize(P, P, n, m, T, P, f2.F32, S),
    "fairy2i_x_digits": lambda: L.fairy2i_x_digits(P, f2.BF16, m, B, P, S),
    "fairy2i_x_digits_f6": lambda: L.fairy2i_x_digits_f6(P, f2.BF16, m, B, P, S),
    "fairy2i_gemv": lambda: L.fairy2i_gemv(P, P, n, m, T, P, f2.BF16, B, P, f2.F32, f2.GEMV_MFMA_BF16, S),
    "fairy2i_gemv_grouped": lambda: L.fairy2i_gemv_grouped(items, 1, m, T, f2.BF16, B, f2.F32, f2.GEMV_VALU, S),
    "fairy2i_gemv_strided": lambda: L.fairy2i_gemv_strided(P, 4096, P, 0, n, m, T, P, f2.BF16, B, P, 2 * n * B, f2.F32,
                                                           2, f2.GEMV_MFMA_BF16, S),
    "fairy2i_act_quant": lambda: L.fairy2i_act_quant(P, f2.BF16, N, 2 * m, P, P, S),
    "fairy2i_gemm": lambda: L.fairy2i_gemm(P, P, n, m, T, P, f2.BF16, P, N, P, f2.F32, P, gws, S),
    "fairy2i_gemm_noalloc": lambda: L.fairy2i_gemm_noalloc(P, P, n, m, T, P, f2.BF16, P, N, P, f2.F32, S),
}
out = {}
for name, call in calls.items():
    status = call()
    out[name] = [status, f2.fairy2i_last_error()]
print(json.dumps(out))
'''


def test_compute_calls_without_a_device_return_err_hip():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + CHILD], env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    out = json.loads(res.stdout.strip().splitlines()[-1])
    if "skipped" in out:
        import pytest
        pytest.skip(out["skipped"])
    import widely_linear_gemv_amd as f2
    assert set(out) >= {n for n in f2.SIGNATURES if n.endswith(("quantize", "quantize_bf16", "quantize_tensor",
                                                               "pack", "dequantize", "x_digits", "x_digits_f6",
                                                               "gemv", "gemv_grouped", "gemv_strided",
                                                               "act_quant", "gemm", "gemm_noalloc"))}
    for name, (status, msg) in out.items():
        assert status == 7, (name, status, msg)          # FAIRY2I_ERR_HIP
        assert msg, name
