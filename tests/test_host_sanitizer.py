"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-sanitized variant of the library (device code as in the normal build, host half of
every source instrumented; `python -m widely_linear_gemv_amd.build --host-san`), then runs the
no-GPU ABI and binding tests against it in a child process with the sanitizer runtime preloaded.
Any invalid host access or undefined behaviour in the argument checks, size arithmetic or error
reporting aborts the child, and the test fails with its report."""
import os
import shutil
import subprocess
import sys

import pytest

from widely_linear_gemv_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC),
                                reason="hipcc not available")


def _stale() -> bool:
    if not os.path.exists(build.SAN_LIB):
        return True
    t = os.path.getmtime(build.SAN_LIB)
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)]
    srcs += [os.path.join(build.INCLUDE, f) for f in os.listdir(build.INCLUDE)]
    return any(os.path.getmtime(p) > t for p in srcs)


@pytest.fixture(scope="module")
def san_env():
    if _stale():
        build.build(host_san=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=build.asan_runtime(), FAIRY2I_LIB=build.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONDONTWRITEBYTECODE="1")
    return env


def run(env, args, timeout=600):
    res = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=timeout)
    return res.returncode, res.stdout + res.stderr


def test_sanitized_library_is_the_one_loaded(san_env):
    code = ("import ctypes, widely_linear_gemv_amd as f2; f2.lib(); "
            "maps = open('/proc/self/maps').read(); "
            "assert f2.LIB_PATH in maps, 'sanitized library not mapped'; "
            "assert hasattr(ctypes.CDLL(None), '__asan_init'), 'sanitizer runtime not loaded'; "
            "print('ok', f2.fairy2i_abi_version())")
    rc, out = run(san_env, ["-c", code])
    assert rc == 0 and "ok" in out, out


def test_abi_and_binding_checks_under_sanitizers(san_env):
    rc, out = run(san_env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            "tests/test_abi_host.py", "tests/test_binding_checks.py"])
    assert rc == 0, out[-6000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
