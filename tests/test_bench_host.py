"""Host logic of bench.py (no GPU): the stored rocprofv3 counter summaries are
reported only for the workload and kernel source they were taken on, the
per-n counter bandwidth is bytes over time, and a run on more than one GPU is
refused."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def write(path, obj):
    with open(path, "w") as f:
        json.dump(obj, f)


def test_stored_traffic_only_for_its_workload_and_source(tmp_path, monkeypatch):
    f = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    sha = bench.kernel_source_hash()
    write(f, {"workload": "fused_qkv_14336x5120 n=16", "kernel_source_sha256_16": sha,
              "hbm_bytes_per_launch": 43196762})
    assert bench.stored_traffic("fused_qkv_14336x5120 n=16") == 43196762
    assert bench.stored_traffic("fused_qkv_14336x5120 n=8") is None          # another n
    assert bench.stored_traffic("ssm_qkvz_16384x5120 n=16") is None          # another shape
    write(f, {"workload": "fused_qkv_14336x5120 n=16", "kernel_source_sha256_16": "0" * 16,
              "hbm_bytes_per_launch": 43196762})
    assert bench.stored_traffic("fused_qkv_14336x5120 n=16") is None         # kernel changed since
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "absent.json"))
    assert bench.stored_traffic("fused_qkv_14336x5120 n=16") is None


def test_counter_bandwidth_per_n(tmp_path, monkeypatch):
    f = tmp_path / "per_n.json"
    monkeypatch.setattr(bench, "PER_N_COUNTERS_FILE", str(f))
    write(f, {"workload": "fused_qkv_14336x5120", "kernel_source_sha256_16": bench.kernel_source_hash(),
              "hbm_bytes_per_launch": {"1": 4_000_000, "16": 8_000_000}})
    sweep = {"1": {"us": 2.0}, "2": {"us": 2.0}, "16": {"us": 4.0}}
    bench.annotate_counter_bandwidth(sweep, "fused_qkv_14336x5120")
    assert sweep["1"]["hbm_GBps_counters"] == 2000.0
    assert sweep["16"]["hbm_GBps_counters"] == 2000.0
    assert sweep["16"]["frac_hbm_peak_counters"] == 0.25
    assert "hbm_GBps_counters" not in sweep["2"]                              # no counters for n = 2
    other = {"16": {"us": 4.0}}
    bench.annotate_counter_bandwidth(other, "ssm_qkvz_16384x5120")
    assert "hbm_GBps_counters" not in other["16"]


def test_committed_counter_summaries_describe_themselves():
    for name in ("gemv_fused_qkv_14336x5120_n16_counters.json",
                 "gemv_fused_qkv_14336x5120_per_n_counters.json"):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            c = json.load(f)
        assert c["workload"].startswith("fused_qkv_14336x5120")
        assert len(c["kernel_source_sha256_16"]) == 16
        assert 0.9 < c["copy_calibration_fetch_factor"] * 2 < 1.1   # a copy reads FETCH_SIZE of half its bytes


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
