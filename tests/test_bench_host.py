"""bench.py's host logic, on the CPU: the one-GPU refusal, the algorithmic
work it divides by, and the traffic record (counter CSVs -> calibrated bytes
-> lookup keyed on the library's sources)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from causal_convolution_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_c4_work_per_launch():
    w = wl.WORKLOADS["c4"]
    P = 81 * 720 * 1280
    assert w.positions == P
    fa, fb = bench.conv_flops(w)
    # 2 P Cout 27 Cin for each conv: 3.715e13, the figure quoted per launch
    assert fa == fb == 2.0 * P * 96 * 27 * 96
    assert abs(fa - 3.715e13) / 3.715e13 < 1e-3
    n1, n2 = bench.norm_bytes(w, 2)
    assert n1 == n2 == 2.0 * P * 96 * 2          # read x once, write y once (28.7 GB)


def test_c5_shortcut_flops_follow_where_it_runs():
    w = wl.WORKLOADS["c5"]
    fa, fb_in = bench.conv_flops(w, shortcut_in_conv=True)
    _, fb_gemm = bench.conv_flops(w, shortcut_in_conv=False)
    # the 1x1x1 product counts toward conv B only when it runs in conv B's K loop
    assert fb_in - fb_gemm == 2.0 * w.positions * w.cout * w.cin


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_calibrates_and_is_keyed_on_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gib = 1 << 30
    # the run's 1 GiB copy reads FETCH_SIZE = half its bytes in KiB and WRITE_SIZE = all of them;
    # small set-up copies go through the same kernel and must not enter the calibration
    fetch = [("__amd_rocclr_copyBuffer", gib / 2048), ("__amd_rocclr_copyBuffer", 3.0),
             ("void conv3d_bf16_kernel<4, 1, 3, 3, 1>(Args)", 1000.0),
             ("void conv3d_bf16_kernel<4, 1, 3, 3, 3>(Args)", 3000.0),
             ("void rmsnorm_silu_kernel<...>(...)", 500.0)]
    write = [("__amd_rocclr_copyBuffer", gib / 1024), ("__amd_rocclr_copyBuffer", 1.0),
             ("void conv3d_bf16_kernel<4, 1, 3, 3, 1>(Args)", 700.0),
             ("void conv3d_bf16_kernel<4, 1, 3, 3, 3>(Args)", 900.0),
             ("void rmsnorm_silu_kernel<...>(...)", 500.0)]
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", write)
    bench.record_traffic("c4", str(tmp_path / "f"), str(tmp_path / "w"), gib)
    t = json.load(open(tmp_path / "traffic.json"))
    e = t["workloads"]["c4"]
    assert e["calibration"]["fetch_factor"] == pytest.approx(2.0, rel=1e-3)
    assert e["calibration"]["write_factor"] == pytest.approx(1.0, rel=1e-3)
    # per launch: the average over the conv dispatches, times 1024, times the factor
    assert e["conv"]["read_bytes"] == pytest.approx(2000.0 * 1024 * 2.0, rel=1e-3)
    assert e["conv"]["write_bytes"] == pytest.approx(800.0 * 1024, rel=1e-3)
    assert bench.measured_traffic("c4", "conv") == pytest.approx((4000.0 + 800.0) * 1024, rel=1e-3)
    assert bench.measured_traffic("c2", "conv") is None          # not recorded
    # another library source -> the record no longer applies
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("c4", "conv") is None


def test_library_sources_cover_every_csrc_file_and_the_build_flags():
    rels = bench.library_sources()
    assert "causal_convolution_amd/build.py" in rels
    for d in ("causal_convolution_amd/csrc", "include"):
        for f in os.listdir(os.path.join(ROOT, d)):
            assert f"{d}/{f}" in rels
