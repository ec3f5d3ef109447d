"""bench.py's host logic on the CPU: the algorithmic byte counts it divides by, the committed
traffic summary it reads (and refuses once the kernel source changed), the host description of the
CPU baseline, and the single-GPU guard."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_gemv_bytes_per_layer(bench):
    # codes T n m / 2 + fp32 scales 16 n T + bf16 x 4 m B + fp32 y 8 n B at n = m = 2048, T = 2
    assert bench.gemv_bytes(2048, 2048, 2, 1) == 2 * 2048 * 2048 // 2 + 16 * 2048 * 2 + 4 * 2048 + 8 * 2048
    assert bench.gemv_bytes(2048, 2048, 2, 1) == 4284416
    assert bench.gemv_bytes(2048, 2048, 2, 4) == 4358144
    assert bench.gemv_bytes(2048, 2048, 2, 16) == 4653056


def test_traffic_summary_is_read_while_the_kernel_is_unchanged(bench, tmp_path, monkeypatch):
    per_layer = bench.measured_traffic_per_layer()
    text = open(os.path.join(ROOT, bench.TRAFFIC_PROFILE)).read()
    total = int(text.split("traffic_bytes_per_launch:")[1].split()[0])
    layers = int(text.split("layers_per_launch:")[1].split()[0])
    assert per_layer == pytest.approx(total / layers)
    # within 1 % of the algorithmic bytes of a batch-1 layer: no re-reads
    assert abs(per_layer / bench.gemv_bytes(2048, 2048, 2, 1) - 1) < 0.01
    # a summary taken for other source text is refused
    stale = tmp_path / "stale.md"
    lines = [ln if "sha256" not in ln else ln.rsplit(" ", 1)[0] + " " + "0" * 64 for ln in text.splitlines()]
    stale.write_text("\n".join(lines))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(stale))
    assert bench.measured_traffic_per_layer() is None


def test_host_info_fields(bench):
    info = bench.host_info()
    assert set(info) >= {"cpu_count", "affinity", "model", "blas_threads"}
    assert info["cpu_count"] == os.cpu_count()


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr and res.stdout == ""
