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


def _counter_csv(path, counter, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
            "Counter_Value"]
    lines = [",".join(cols)]
    for i, (name, v) in enumerate(rows):
        lines.append(f'{i},{i},256,"{name}",{counter},{v}')
    path.write_text("\n".join(lines) + "\n")


def test_traffic_summary_scales_by_the_copy(tmp_path):
    """Counters in KiB per dispatch, scaled so the 256 MiB calibration copy
    reads and writes 256 MiB: a copy that reads 128 Ki 'KiB' gives a read
    scale of 2; the GEMM dispatches are split, in dispatch order, into one
    equal block per counter workload, and each block's bytes are averaged."""
    ns = "void mixq::(anonymous namespace)::"
    g8 = ns + "gemm_kernel<256, 256, 2, 2, 8, 4, 6, false, false, false>(mixq::GemmArgs)"
    g4 = ns + "gemm_kernel<256, 256, 2, 2, 4, 2, 4, false, false, false>(mixq::GemmArgs)"
    g1 = ns + "gemm_kernel<128, 128, 2, 2, 8, 4, 5, false, false, false>(mixq::GemmArgs)"
    gq = ns + "gate_quant_kernel<4, 4, false, false>(mixq::ActArgs)"
    cp = "__amd_rocclr_copyBuffer"
    assert bench.COUNTER_WORKLOADS == ("prefill_w8", "prefill_w4", "llama7b_up", "llama70b_up",
                                       "decode_seq")
    # the workloads' GEMMs, two dispatches each, in the order they ran:
    # llama70b_up reuses the prefill kernel, decode_seq llama7b_up's
    f_g = [(g8, 100000), (g8, 102000), (g4, 80000), (g4, 80000), (g1, 38000), (g1, 38000),
           (g8, 150000), (g8, 150000), (g1, 45000), (g1, 46000)]
    w_g = [(g8, 65536), (g8, 65536), (g4, 65536), (g4, 65536), (g1, 22016), (g1, 22016),
           (g8, 229376), (g8, 229376), (g1, 24000), (g1, 24000)]
    fe, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    # three calibration copies first; a later (smaller) copy is not one of them
    _counter_csv(fe, "FETCH_SIZE", [(cp, 131072)] * 3 + [(cp, 50), (gq, 16000)] + f_g)
    _counter_csv(wr, "WRITE_SIZE", [(cp, 262144)] * 3 + [(cp, 9)] + w_g)
    oj, ot = tmp_path / "t.json", tmp_path / "t.txt"
    bench.traffic_summary(str(fe), str(wr), str(oj), str(ot))
    t = json.loads(oj.read_text())
    assert t["gemm_source_sha"] == bench.gemm_source_sha()
    w8 = t["workloads"]["prefill_w8"]
    assert w8["read_scale"] == 2.0 and w8["write_scale"] == 1.0 and w8["dispatches"] == 2
    assert w8["hbm_bytes_per_launch"] == 101000 * 1024 * 2 + 65536 * 1024
    assert t["workloads"]["prefill_w4"]["hbm_bytes_per_launch"] == 80000 * 2048 + 65536 * 1024
    assert t["workloads"]["llama70b_up"]["hbm_bytes_per_launch"] == 150000 * 2048 + 229376 * 1024
    assert t["workloads"]["decode_seq"]["hbm_bytes_per_launch"] == 45500 * 2048 + 24000 * 1024
    assert "gate_quant_kernel<4, 4, false, false> (1 dispatches)" in ot.read_text()
    assert bench.kernel_short_name(g8) == "gemm_kernel<256, 256, 2, 2, 8, 4, 6, false, false, false>"
    # a block that mixes two kernels, or a count that does not divide, is refused
    with pytest.raises(SystemExit):
        bench.gemm_blocks([("a", 1), ("b", 1)], ("x",))
    with pytest.raises(SystemExit):
        bench.gemm_blocks([("a", 1)] * 3, ("x", "y"))


def test_trace_summary_windows(tmp_path):
    """The headline GEMM's clean- and hot-cache windows are the last 100 of
    each run of at least 200 consecutive dispatches of that kernel; shorter
    runs (the timed steps, where the activation kernels interleave) are not."""
    ns = "void mixq::(anonymous namespace)::"
    g8 = ns + "gemm_kernel<256, 256, 2, 2, 8, 4, 6, false, false, false>(mixq::GemmArgs)"
    gq = ns + "gate_quant_kernel<4, 4, false, false, true, true>(mixq::ActArgs)"
    pr = ns + "mfma_probe_kernel(signed char const*, signed char const*, long, long, int, int*, long*)"
    seq = []
    for i in range(5):                       # steps: act and GEMM interleaved
        seq += [(gq, 10.0), (g8, 300.0)]
    seq += [(g8, 140.0)] * 100 + [(g8, 120.0)] * 100    # clean: per-launch events, back to back
    seq += [(gq, 10.0)]
    seq += [(g8, 150.0)] * 100 + [(g8, 130.0)] * 100    # hot
    seq += [(pr, 90.0)] * 50 + [(pr, 80.0)] * 100
    lines = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    for name, us in seq:
        lines.append(f'"{name}",{t},{t + int(us * 1000)}')
        t += int(us * 1000) + 500
    csvp, out = tmp_path / "t.csv", tmp_path / "s.txt"
    csvp.write_text("\n".join(lines) + "\n")
    bench.trace_summary(str(csvp), str(out))
    text = out.read_text()
    assert "clean-cache window: 100 back-to-back dispatches, avg 120.00 us" in text
    assert "hot-cache window: 100 back-to-back dispatches, avg 130.00 us" in text
    assert "last 100 dispatches, avg 80.00 us" in text
    assert text.splitlines()[1].startswith("gemm_kernel<256, 256, 2, 2, 8, 4, 6, false, false, false>")
