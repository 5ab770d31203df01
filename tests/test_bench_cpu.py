"""bench.py's host logic, on the CPU: the one-GPU contract, the algorithmic
byte count of a GEMM launch, the traffic figure's source check, and the
CPU-baseline record."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixed_precision_quantized_amax_amd import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_headline_launch():
    """Xq 16 MiB + INT8 weight 64 MiB + both scale vectors + the padded
    outlier matrices (82 channels -> 96 columns) + fp32 Y 64 MiB."""
    wl = workloads.WORKLOADS["prefill_w8"]
    assert bench.algorithmic_bytes(wl, 82) == (16 << 20) + (64 << 20) + 4 * 10240 + \
        2 * 96 * 10240 + (64 << 20)
    w4 = workloads.WORKLOADS["prefill_w4"]
    assert bench.algorithmic_bytes(w4, 0) == (16 << 20) + (32 << 20) + 4 * 10240 + (64 << 20)


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    t = tmp_path / "traffic.json"
    t.write_text(json.dumps({"gemm_source_sha": bench.gemm_source_sha(),
                             "workloads": {"prefill_w8": {"hbm_bytes_per_launch": 1234}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(t))
    assert bench.gemm_traffic("prefill_w8") == 1234
    assert bench.gemm_traffic("llama7b_up") is None
    monkeypatch.setattr(bench, "gemm_source_sha", lambda: "0" * 16)
    assert bench.gemm_traffic("prefill_w8") is None


def test_cpu_baseline_record():
    r = bench.run_cpu_baseline(workloads.WORKLOADS["tiny"], target_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TOPS"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "tokens" in r["sample"]
