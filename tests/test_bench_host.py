"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal, the CPU-baseline fields,
and that stored counter traffic is reported only for the kernel source it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_workload  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_before_any_device_work(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_reports_affinity_cores_and_the_oracle_sample():
    w = make_workload(0)
    cb = bench.cpu_baseline(w, 0.2)
    assert cb["kind"] == "oracle"
    assert cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] == len(os.sched_getaffinity(0))
    assert "blas_threads" in cb
    assert "query rows of the same workload" in cb["sample"]


def test_stored_traffic_follows_the_kernel_source_hash(tmp_path, monkeypatch):
    # a counter summary carrying the current hash is read; any other hash is ignored
    prof = tmp_path / "profiles"
    prof.mkdir()
    h = bench.kernel_source_hash(True)
    (prof / "mla_decode_config2_pmc.md").write_text(
        f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 123456789\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic(2, True) == 123456789.0
    (prof / "mla_decode_config2_pmc.md").write_text(
        "kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 123456789\n")
    assert bench.stored_traffic(2, True) is None
    assert bench.stored_traffic(3, False) is None          # no summary for that workload here
