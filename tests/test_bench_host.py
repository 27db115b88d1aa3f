"""Host logic of bench.py (no GPU): the stored rocprofv3 counter summaries are
reported only for the workload and kernel source they were taken on, the
per-n counter bandwidth is bytes over time, the last stdout line stays
compact whatever the detail holds, and a run on more than one GPU is
refused."""
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def write(path, obj):
    with open(path, "w") as f:
        json.dump(obj, f)


def test_stored_traffic_only_for_its_workload_and_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    f = bench.counters_file("ssm_qkvz_16384x5120", 16)
    assert os.path.dirname(f) == str(tmp_path)
    sha = bench.kernel_code_hash()
    write(f, {"workload": "ssm_qkvz_16384x5120 n=16", "kernel_code_sha256_16": sha,
              "hbm_bytes_per_launch": 48700000})
    assert bench.stored_traffic("ssm_qkvz_16384x5120", 16) == 48700000
    assert bench.stored_traffic("ssm_qkvz_16384x5120", 8) is None           # another n: no file
    assert bench.stored_traffic("fused_qkv_14336x5120", 16) is None         # another shape: no file
    write(f, {"workload": "fused_qkv_14336x5120 n=16", "kernel_code_sha256_16": sha,
              "hbm_bytes_per_launch": 48700000})
    assert bench.stored_traffic("ssm_qkvz_16384x5120", 16) is None          # file describes another workload
    write(f, {"workload": "ssm_qkvz_16384x5120 n=16", "kernel_code_sha256_16": "0" * 16,
              "hbm_bytes_per_launch": 48700000})
    assert bench.stored_traffic("ssm_qkvz_16384x5120", 16) is None          # kernel changed since


def test_counter_bandwidth_per_n(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    write(bench.per_n_counters_file("fused_qkv_14336x5120"),
          {"workload": "fused_qkv_14336x5120", "kernel_code_sha256_16": bench.kernel_code_hash(),
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
    names = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith("_counters.json")]
    for name in names:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            c = json.load(f)
        shape = re.match(r"gemv_(.+?)_(n\d+|per_n)_counters\.json$", name).group(1)
        assert c["workload"].startswith(shape), name
        assert len(c["kernel_code_sha256_16"]) == 16
        assert 0.9 < c["copy_calibration_fetch_factor"] * 2 < 1.1   # a copy reads FETCH_SIZE of half its bytes


def _fake_result():
    point = {"us": 9.5, "p10_us": 9.4, "p50_us": 9.5, "p90_us": 9.7, "weight_GBps": 4900.0,
             "frac_hbm_peak": 0.61, "gemv_tokens_per_s": 1.0e6, "t_over_t1": 1.1, "warm_us": 9.0}
    sweep = {str(n): dict(point) for n in range(1, 17)}
    r = {"metric": bench.METRIC, "value": 4000.0, "unit": "GB/s", "n_gpus": 1, "steps": 400, "warmup": 50,
         "ms_per_step": 0.0115, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
         "dtype": "bf16", "data": "synthetic " * 20,
         "config": {"workload": "ssm_qkvz_16384x5120", "N": 16384, "K": 5120, "n_tokens": 16,
                    "entry": "nvfp4_gemv", "launch": {"workgroups": 256, "waves_per_workgroup": 8,
                                                      "tiles_per_wave": 5},
                    "rotation_alloc": "torch", "timing": "x" * 120},
         "frac_hbm_peak": 0.5, "gemv_tokens_per_s": 1.4e6,
         "per_call_us_over_replays": {"p10": 11.4, "p50": 11.5, "p90": 11.6, "replays": 7,
                                      "launches_per_replay": 50},
         "roofline": {"bound": "hbm", "achieved": 4100.0, "peak": 8000.0, "unit": "GB/s", "frac": 0.51,
                      "traffic": 48700000, "kernel": "nvfp4_gemv_kernel<5, 4, true, false, false>",
                      "algorithmic_bytes_per_launch": 47874560},
         "context_pages": bench.PAGES_CONTEXT,
         "sweep": {name: sweep for name in bench.TARGET_SHAPES},
         "extra_shapes": {"x": {"sweep": sweep}}, "prefill_fused_qkv": {str(n): point for n in bench.PREFILL_N},
         "decode_step": {"us_per_step": 700.0, "frac_hbm_peak": 0.52},
         "launch_ramp": {"empty_launch_us_256wg": 1.6, "read_1GiB_us": 170.0, "read_1GiB_GBps": 6300.0,
                         "read_1GiB_frac_hbm_peak": 0.79,
                         "ssm_qkvz_16384x5120": {"read_us": 8.1, "read_frac_hbm_peak": 0.72,
                                                 "streaming_us_at_1GiB_rate": 7.5, "fixed_us": 0.6}},
         "cpu_baseline": {"value": 0.8, "unit": "effective weight GB/s", "gemv_tokens_per_s": 270.0,
                          "cores": 16, "kind": "oracle", "sample": "s" * 100,
                          "single_thread": {"value": 0.05}, "n1": {"value": 1.0}, "host": {"cpu_model": "c"}}}
    r["targets"] = bench.targets(r["sweep"], r["decode_step"])
    return r


def test_last_line_is_compact_and_complete():
    r = _fake_result()
    s = bench.summarize(r)
    line = json.dumps(s)
    assert len(line) <= bench.SUMMARY_MAX_BYTES, len(line)
    assert len(json.dumps({"bench_detail": r})) > len(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in s, key
    assert s["config"]["workload"] == "ssm_qkvz_16384x5120"
    assert set(s["cpu_baseline"]) >= {"value", "unit", "cores", "kind", "sample"}
    assert set(s["roofline"]) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    for name in bench.TARGET_SHAPES:
        assert set(s["targets"][name]) == {"n1", "n16", "us"}
    assert "sweep" not in s and "prefill_fused_qkv" not in s


def test_default_workload_is_the_largest_single_projection():
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="ssm_qkvz_16384x5120"' in src
    assert bench.SHAPES["ssm_qkvz_16384x5120"] == (16384, 5120)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
