#!/usr/bin/env python3
"""Benchmark of the NVFP4 decode projection on one MI355X.

Workload (default): the fused attention QKV projection, W 14336 x 5120 NVFP4
(q|k|v = 8192|3072|3072 rows, written straight to per-projection offsets),
x bf16 N(0,1), n = 16 decode tokens per step.  A step is one projection of
the whole token batch (one nvfp4_gemv_qkv call).  Weights are synthetic
(N(0, 0.02) fp32 quantised on the GPU with the library's quantiser), one
distinct copy per rotation slot, with enough copies (>= 1 GiB) that the 256 MB
Infinity Cache cannot serve them: every call reads its weight from HBM.

Timing: W warm-up steps, then exactly K steps replayed from a HIP graph
(launches back-to-back on one stream, no host launch overhead) between two
device synchronisations, timed with HIP events on that stream.

Printed: one JSON line with the headline metric (effective weight GB/s =
N*K*9/16 bytes per call / time per call), GEMV-tokens/s, a per-n sweep
(n = 1, 2, 3, 4, 8, 16), the roofline of the GEMV kernel and the CPU oracle's
rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

SHAPES = {
    "fused_qkv_14336x5120": (14336, 5120),
    "ssm_qkvz_16384x5120": (16384, 5120),
    "ssm_out_proj_5120x6144": (5120, 6144),
    "smoke_1024x1024": (1024, 1024),
}
QKV_ROWS = (8192, 3072, 3072)
ROTATION_BYTES = 1 << 30
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemv_fused_qkv_14336x5120_n16_counters.json")
KERNEL_SOURCE = os.path.join(ROOT, "nvfp4_weight_only_02_amd", "csrc", "nvfp4.hip")


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Rotation:
    """Distinct packed copies of one weight shape, totalling >= ROTATION_BYTES."""

    def __init__(self, nv, torch, N, K, seed, min_bytes=ROTATION_BYTES):
        from nvfp4_weight_only_02_amd import metrics
        self.N, self.K = N, K
        wb = metrics.weight_bytes(N, K)
        self.count = max(2, math.ceil(min_bytes / wb))
        self.copies = []
        gen = torch.Generator(device="cuda")
        for c in range(self.count):
            gen.manual_seed(seed + c)
            W = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
            self.copies.append(nv.PackedWeight.from_float(W))
            del W
        torch.cuda.synchronize()


def make_x(torch, n, K, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn((n, K), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


_hip = None


def graph_upload(torch, g):
    """Upload an instantiated graph to the device (hipGraphUpload) so its
    first replay does not pay the upload inside a timed region."""
    global _hip
    import ctypes
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipGraphUpload.restype = ctypes.c_int
        _hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    st = _hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError("hipGraphUpload failed (%d)" % st)
    torch.cuda.synchronize()


def capture(torch, fn, launches):
    """HIP graph of `launches` calls fn(i) on torch's capture stream, uploaded."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(i)
    graph_upload(torch, g)
    return g


def copy_calibration(torch, mib=256, reps=5):
    """A plain device copy of known size (for scaling the FETCH_SIZE and
    WRITE_SIZE counters): each copy reads and writes exactly `mib` MiB."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes": mib << 20, "copies": reps}


def time_graph(torch, g, replays):
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(replays):
        g.replay()
    e1.record(s)
    e1.synchronize()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def sweep_shape(nv, torch, metrics, rot, n_list, call, launches_per_graph, replays):
    out = {}
    wb = metrics.weight_bytes(rot.N, rot.K)
    for n in n_list:
        X = make_x(torch, n, rot.K, 2000 + n)
        Y = torch.empty((n, rot.N), dtype=torch.bfloat16, device="cuda")
        g = capture(torch, lambda i: call(rot.copies[i % rot.count], X, Y), launches_per_graph)
        g.replay()
        t = time_graph(torch, g, replays) / (launches_per_graph * replays)
        # warm reference: the same weight copy on every call (served by the caches)
        gw = capture(torch, lambda i: call(rot.copies[0], X, Y), 32)
        gw.replay()
        tw = time_graph(torch, gw, 4) / 128
        out[str(n)] = {
            "us": round(t * 1e6, 3),
            "weight_GBps": round(wb / t / 1e9, 1),
            "frac_hbm_peak": round(wb / t / 1e9 / metrics.HBM_PEAK_GBPS, 4),
            "gemv_tokens_per_s": round(n / t, 1),
            "t_over_t1": None,
            "warm_us": round(tw * 1e6, 3),
        }
        del g, gw
    t1 = out[str(n_list[0])]["us"] if n_list[0] == 1 else None
    for n in n_list:
        if t1:
            out[str(n)]["t_over_t1"] = round(out[str(n)]["us"] / t1, 3)
    return out


def cpu_baseline(N, K, n, seconds):
    """The oracle (fp64, OpenMP over rows) on the same workload shape: the
    whole N x K weight for n tokens, repeated until `seconds` of CPU time."""
    import numpy as np
    import oracle as O
    from nvfp4_weight_only_02_amd import inputs, metrics
    W = inputs.weights_f32(N, K, inputs.weight_seed(1))
    codes, scales, g = O.quantize(W)
    X = inputs.activations_bf16(n, K, inputs.act_seed(1, n))
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        O.gemv(codes, scales, g, X)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= seconds and len(times) >= 2:
            break
    t = float(np.median(times))
    wb = metrics.weight_bytes(N, K)
    return {
        "value": round(wb / t / 1e9, 4),
        "unit": "effective weight GB/s",
        "gemv_tokens_per_s": round(n / t, 2),
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": "full %dx%d NVFP4 weight, n=%d tokens, %d runs, median %.3f s per call"
                  % (N, K, n, len(times), t),
    }


def stored_traffic(launch_bytes):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None if the summary is absent or was taken on a different kernel."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--n", type=int, default=16)
    ap.add_argument("--workload", default="fused_qkv_14336x5120", choices=sorted(SHAPES))
    ap.add_argument("--sweep", default="1,2,3,4,8,16", help="token counts of the per-n sweep ('' = none)")
    ap.add_argument("--all-shapes", action="store_true", help="also sweep ssm_qkvz, ssm_out_proj and the decode-step set")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="only the timed region (for rocprofv3 runs): no sweep, no CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_weight_only_02_amd as nv
    from nvfp4_weight_only_02_amd import metrics

    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_weight_only_02_amd import build as b
        b.build()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch)), flush=True)
        return
    N, K = SHAPES[args.workload]
    n = args.n
    qkv = args.workload.startswith("fused_qkv")

    log("building rotation of %s copies ..." % args.workload)
    rot = Rotation(nv, torch, N, K, seed=1100)
    log("rotation: %d copies, %.2f GiB" % (rot.count, rot.count * metrics.weight_bytes(N, K) / 2**30))

    if qkv:
        offs = (0, QKV_ROWS[0], QKV_ROWS[0] + QKV_ROWS[1])

        def call(w, X, Y):
            nv.gemv_qkv(w, X, QKV_ROWS, offs, N, out=Y)
    else:
        def call(w, X, Y):
            nv.gemv(w, X, out=Y)

    X = make_x(torch, n, K, 2000 + n)
    Y = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
    # The K timed steps replay one graph of L launches K/L times (L the
    # largest divisor of K up to 64; very long graphs add per-node overhead).
    L = max(d for d in range(1, min(args.steps, 64) + 1) if args.steps % d == 0)
    gt = capture(torch, lambda i: call(rot.copies[i % rot.count], X, Y), L)
    # Warm-up: W steps, as whole replays of the timed graph itself (its first
    # replay costs more than the others) plus a remainder graph.
    if args.warmup % L:
        gw = capture(torch, lambda i: call(rot.copies[i % rot.count], X, Y), args.warmup % L)
        gw.replay()
    for _ in range(args.warmup // L):
        gt.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_host0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps // L):
        gt.replay()
    e1.record(s)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    elapsed = e0.elapsed_time(e1) * 1e-3
    t_call = elapsed / args.steps

    wb = metrics.weight_bytes(N, K)
    ab = metrics.algorithmic_bytes(n, N, K)
    value = wb / t_call / 1e9
    wg, waves, tpw = nv.launch_geometry(n, N, K)
    result = {
        "metric": "effective weight GB/s (NVFP4 weight bytes N*K*9/16 per call / time per call)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_call * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 weights (e2m1 + e4m3 block scale), bf16 activations, fp32 accumulate",
        "data": "synthetic: W ~ N(0,0.02) fp32 quantised on the GPU, x ~ N(0,1) bf16; %d distinct weight copies rotated (%.2f GiB, cold against the 256 MB Infinity Cache)" % (rot.count, rot.count * wb / 2**30),
        "config": {"workload": args.workload, "N": N, "K": K, "n_tokens": n,
                   "qkv_rows": list(QKV_ROWS) if qkv else None,
                   "launch": {"workgroups": wg, "waves_per_workgroup": waves, "tiles_per_wave": tpw},
                   "timing": "%d replays of a HIP graph of %d back-to-back launches, HIP events on the launch stream" % (args.steps // L, L)},
        "frac_hbm_peak": round(value / metrics.HBM_PEAK_GBPS, 4),
        "gemv_tokens_per_s": round(n / t_call, 1),
        "host_wall_s_timed_region": round(t_host, 6),
        "roofline": {
            "bound": "hbm",
            "achieved": round(ab / t_call / 1e9, 1),
            "peak": metrics.HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(ab / t_call / 1e9 / metrics.HBM_PEAK_GBPS, 4),
            "traffic": stored_traffic(ab),
            "kernel": "nvfp4_gemv_kernel<%d,%d,%s>" % (waves, tpw, "true" if K % 128 == 0 else "false"),
            "algorithmic_bytes_per_launch": ab,
        },
    }

    if not args.profile_only:
        n_list = [int(v) for v in args.sweep.split(",") if v.strip()]
        if n_list:
            log("per-n sweep ...")
            result["sweep"] = {args.workload: sweep_shape(nv, torch, metrics, rot, n_list, call,
                                                          2 * rot.count, 4)}
            # warm-cache reference: the same weight copy every call
            Xw = make_x(torch, n, K, 77)
            Yw = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
            gww = capture(torch, lambda i: call(rot.copies[0], Xw, Yw), 64)
            gww.replay()
            tw = time_graph(torch, gww, 4) / 256
            result["warm_same_weight"] = {"n": n, "us": round(tw * 1e6, 3),
                                          "weight_GBps": round(wb / tw / 1e9, 1)}
        if args.all_shapes:
            del rot, gt
            torch.cuda.empty_cache()
            for name in ("ssm_qkvz_16384x5120", "ssm_out_proj_5120x6144"):
                log("sweep", name)
                N2, K2 = SHAPES[name]
                r2 = Rotation(nv, torch, N2, K2, seed=3100)
                result["sweep"][name] = sweep_shape(
                    nv, torch, metrics, r2, n_list or [1, 16],
                    lambda w, X, Y: nv.gemv(w, X, out=Y), 2 * r2.count, 4)
                del r2
                torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            log("cpu baseline ...")
            result["cpu_baseline"] = cpu_baseline(N, K, n, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
