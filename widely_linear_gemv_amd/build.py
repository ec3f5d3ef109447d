"""Build libfairy2i.so in-tree with hipcc for gfx950.

    python -m widely_linear_gemv_amd.build              # or: python widely_linear_gemv_amd/build.py
    python -m widely_linear_gemv_amd.build --host-san   # host-sanitized variant (see below)

Each HIP source compiles to an object in _build/, then one shared library is linked next
to this file.  Always recompiles (it is the "does it build" check as well as the build).

The host-sanitized variant instruments the host half of every source (the C ABI's argument
checks, size arithmetic and launch set-up) with AddressSanitizer and UndefinedBehaviorSanitizer;
device code is compiled exactly as in the normal build.  It is linked to
_build/host-san/libfairy2i.so without a sanitizer runtime: load it into a process that has the
runtime preloaded (LD_PRELOAD=<clang>/lib/linux/libclang_rt.asan-x86_64.so) and point the
binding at it with FAIRY2I_LIB.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfairy2i.so")
C_DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "driver.c")
C_DRIVER = os.path.join(ROOT, "tests", "c_abi", "fairy2i_c_driver")
SAN_BUILD = os.path.join(BUILD, "host-san")
SAN_LIB = os.path.join(SAN_BUILD, "libfairy2i.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-I", INCLUDE, "-I", CSRC,
    # device code: no packed fp32 instructions (the host pass warns that it does not know it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-command-line-argument",
]
# Sources whose fp64/fp32 results must match the CPU reference bit for bit get no contraction.
SOURCES = {
    "quantize.hip": ["-ffp-contract=off"],
    "gemv_valu.hip": [],
    "gemv_mfma.hip": [],
    "gemv_i8.hip": [],
    "gemv_f4.hip": [],
    "gemv_f8x.hip": [],
    "prefill.hip": ["-ffp-contract=off"],
    "dequant.hip": ["-ffp-contract=off"],
    "api.cpp": ["-x", "hip"],
}


# Host-only instrumentation: each flag goes to the host compilation alone.
HOST_SAN = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def _compile(src: str, extra: list[str], out_dir: str = BUILD, host_flags: tuple = ()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *host_flags, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, host_san: bool = False) -> str:
    out_dir, lib_path = (SAN_BUILD, SAN_LIB) if host_san else (BUILD, LIB)
    flags = tuple(HOST_SAN) if host_san else ()
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], out_dir, flags), SOURCES.items()))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def build_c_driver(verbose: bool = False) -> str:
    """The plain-C driver of the ABI used by the tests (host code only, built with gcc against
    include/fairy2i.h and the in-tree library)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cc = shutil.which("gcc") or shutil.which("cc") or "gcc"
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), C_DRIVER_SRC, "-L", PKG, "-lfairy2i",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../widely_linear_gemv_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", C_DRIVER]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C driver build failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {C_DRIVER}")
    return C_DRIVER


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime that the host-sanitized library needs preloaded."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(clang)) if os.path.isdir(clang) else []:
        cand = os.path.join(clang, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return os.path.realpath(cand)
    raise RuntimeError("AddressSanitizer runtime libclang_rt.asan-x86_64.so not found")


if __name__ == "__main__":
    san = "--host-san" in sys.argv[1:]
    build(verbose=True, host_san=san)
    if not san:
        build_c_driver(verbose=True)
    sys.exit(0)
