#!/usr/bin/env python3
"""Benchmark of the NVFP4 decode projection on one MI355X.

Headline workload (the last stdout line): the ssm_qkvz projection, W 16384 x
5120 NVFP4, x bf16 N(0,1) with each token row scaled by U(0.5, 2), n = 16
decode tokens per step; a step is one projection of the whole token batch (one
nvfp4_gemv call).  This is the largest single projection of the pages'
decode-shape table (spark_model::layers page, doc comment of w4a16_k64_min_k,
measured at M = 16).  Weights are synthetic (N(0, 0.02) fp32 quantised on the
GPU with the library's quantiser), one distinct copy per rotation slot, with
enough copies (>= 1 GiB) that the 256 MB Infinity Cache cannot serve them:
every call reads its weight from HBM.

Timing: after building the weights, the timed graph is replayed untimed for
a settle period (the quantiser's fp64 kernels leave the GPU below its steady
clock for ~10 ms), then W warm-up steps, then exactly K steps replayed from a
HIP graph (launches back-to-back on one stream, no host launch overhead)
between two device synchronisations, timed with HIP events on that stream.

Output: the full results as one JSON line ({"bench_detail": ...}, also written
to --detail-out), then, as the LAST line, a compact summary of a few KB: the
headline, its roofline, the CPU oracle baseline, the per-shape target
fractions and the launch-ramp figures.

Also measured (default; --quick skips them):
  * per-n sweep n = 1..16 of every decode shape (ssm_qkvz with per-token row
    scales, fused QKV through both entry points, ssm_out_proj), cold and
    warm, each point with the p10 / p50 / p90 of its replays;
  * token-tile schedules on ssm_qkvz: the pages' greedy 3-token tiling
    against one launch for all tokens, for every n;
  * ssm_out_proj with 1% all-zero blocks and 1% 50x-rms outliers;
  * the decode-step sweep: 48 distinct ssm_qkvz + 16 distinct fused-QKV
    matrices (2.93 GB) back to back on one stream at n = 16;
  * the launch ramp: the cost of an empty launch of the GEMV's shape, the
    read ceiling of each shape's bytes (libnvfp4_probes, same rotation), and
    the streaming rate of one 1 GiB read;
  * shapes beyond the decode projections (dense FFN gate+up and down with
    K > 8192, the latter also in K parts through nvfp4_gemv_ws, the pages'
    small hidden-2048 attention layer) at n = 1..16;
  * the MFMA-vs-VALU arithmetic probe and the prefill GEMM (nvfp4_gemm) on the
    fused QKV weight at n = 32..2048;
  * the CPU oracle on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

SHAPES = {
    "ssm_qkvz_16384x5120": (16384, 5120),
    "fused_qkv_14336x5120": (14336, 5120),
    "ssm_out_proj_5120x6144": (5120, 6144),
    "dense_ffn_down_5120x17408": (5120, 17408),
    "smoke_1024x1024": (1024, 1024),
}
# The three projection shapes the per-shape targets are stated for.
TARGET_SHAPES = ("ssm_qkvz_16384x5120", "fused_qkv_14336x5120", "ssm_out_proj_5120x6144")
TARGET_BAR = {"n1": 0.75, "n16": 0.65}
QKV_ROWS = (8192, 3072, 3072)
QKV_OFFS = (0, 8192, 11264)
# Shapes beyond the decode projections (name, N, K, fused q|k|v rows or None,
# what it is).  The FFN intermediate size (17408) is a synthetic choice for a
# hidden-5120 dense model; the small attention layer is hidden 2048 with 16
# query heads and 2 KV heads of dimension 256.
EXTRA_SHAPES = [
    ("ffn_gate_up_34816x5120", 34816, 5120, None, "dense FFN gate+up fused, intermediate 17408"),
    ("ffn_down_5120x17408", 5120, 17408, None,
     "dense FFN down: K in 3 chunk passes (nvfp4_gemv), or in K parts (nvfp4_gemv_ws)"),
    ("attn_small_qkv_5120x2048", 5120, 2048, (4096, 512, 512), "hidden 2048: fused q|k|v 4096|512|512"),
    ("attn_small_o_proj_2048x4096", 2048, 4096, None, "hidden 2048: o_proj"),
]
EXTRA_N = [1, 2, 4, 8, 16]
# Prefill (many-token) GEMM sweep on the fused QKV weight.
PREFILL_N = [32, 64, 128, 256, 384, 512, 768, 1024, 2048]
ROTATION_BYTES = 1 << 30
# The pages' own numbers, on another GPU and memory system (GB10, sm_121):
# context for the reader, never a target and never the vs_baseline figure.
PAGES_CONTEXT = {
    "hardware": "GB10 (sm_121), CUDA kernels, as the pages report them",
    "w4a16_tile_gemm_M16_us": {  # spark_model::layers page, measured decode-shape table
        "ssm_qkvz_16384x5120": [272.4, 281.9, 341.6],
        "fused_qkv_14336x5120": [262.8, 273.9, 328.5],
        "ssm_out_proj_5120x6144": [163.3, 237.7, 240.7],
        "stream_ceiling_GBps": 230},
    "decode_tok_s_per_sequence_C4": {"wide_gemm": 15.8, "tiled_gemv": 26.7},  # Atlas PR #266, A/B table
    "note": "different hardware and end-to-end serving numbers; no figure of the pages is this metric on MI355X",
}
METRIC = "effective weight GB/s (% of HBM peak) and GEMV-tokens/s vs n=1..16"
SUMMARY_MAX_BYTES = 4096   # the last stdout line stays within this
SETTLE_S = 0.1
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_LIB = os.path.join(ROOT, "nvfp4_weight_only_02_amd", "libnvfp4.so")


def counters_file(workload: str, n: int) -> str:
    return os.path.join(PROFILES, "gemv_%s_n%d_counters.json" % (workload, n))


def per_n_counters_file(workload: str) -> str:
    return os.path.join(PROFILES, "gemv_%s_per_n_counters.json" % workload)


_CODE_HASH = []


def kernel_code_hash():
    """sha256 prefix of the gfx950 code of every nvfp4_gemv_kernel
    instantiation in the built libnvfp4.so (names and instructions, no
    addresses), which stored counters must match: they were measured on
    exactly that code, and host-side changes to the library leave it as it
    is.  None if the library cannot be disassembled here (then no stored
    figure is used)."""
    if not _CODE_HASH:
        try:
            from nvfp4_weight_only_02_amd import asmcheck
            _CODE_HASH.append(asmcheck.code_hash(KERNEL_LIB))
        except Exception:
            _CODE_HASH.append(None)
    return _CODE_HASH[0]


_T0 = time.perf_counter()


def log(*a):
    print("[%6.1f s]" % (time.perf_counter() - _T0), *a, file=sys.stderr, flush=True)


def zero_outlier_(torch, W, gen, frac=0.01, factor=50.0):
    """In place on a [N, K] fp32 device tensor: two disjoint random 1% sets of
    16-element K-blocks; the first set becomes all zero, in the second one
    uniformly chosen element becomes sign(orig) * factor * rms(orig block)."""
    N, K = W.shape
    Wb = W.view(N * (K // 16), 16)
    nb = Wb.shape[0]
    perm = torch.randperm(nb, generator=gen, device=W.device)
    nz = no = int(round(frac * nb))
    zb, ob = perm[:nz], perm[nz:nz + no]
    pos = torch.randint(0, 16, (no,), generator=gen, device=W.device)
    rms = Wb[ob].double().pow(2).mean(dim=1).sqrt()
    orig = Wb[ob, pos]
    sign = torch.where(orig < 0, -1.0, 1.0).double()
    Wb[zb] = 0.0
    Wb[ob, pos] = (sign * factor * rms).float()
    return W


class _RawBuf:
    """A device address that quacks like a tensor for the binding (data_ptr)."""

    def __init__(self, ptr: int):
        self.ptr = ptr

    def data_ptr(self) -> int:
        return self.ptr


_hip = None


def hip():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMalloc.restype = ctypes.c_int
        _hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
        _hip.hipFree.restype = ctypes.c_int
        _hip.hipFree.argtypes = [ctypes.c_void_p]
        _hip.hipGraphUpload.restype = ctypes.c_int
        _hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return _hip


class Rotation:
    """Distinct packed copies of one weight shape, totalling >= min_bytes.

    alloc: "torch" (every copy its own pair of torch allocations, the
    default), "slab" (one torch allocation, each copy's codes and scales at
    2 MiB-aligned offsets of it) or "hip" (the same slab layout in one
    hipMalloc allocation made here, outside torch's caching allocator)."""

    def __init__(self, nv, torch, N, K, seed, min_bytes=ROTATION_BYTES, count=None,
                 zero_outlier=False, alloc="torch"):
        from nvfp4_weight_only_02_amd import metrics
        self.N, self.K = N, K
        wb = metrics.weight_bytes(N, K)
        self.count = count or max(2, math.ceil(min_bytes / wb))
        self.copies = []
        self.alloc = alloc
        self._slab = None
        self._hip_ptr = None
        cb, sb = nv.packed_codes_bytes(N, K), nv.packed_scales_bytes(N, K)
        align = 2 << 20
        cpad, spad = -(-cb // align) * align, -(-sb // align) * align
        if alloc == "slab":
            self._slab = torch.empty(self.count * (cpad + spad), dtype=torch.uint8, device="cuda")
            base = self._slab.data_ptr()
        elif alloc == "hip":
            p = ctypes.c_void_p()
            st = hip().hipMalloc(ctypes.byref(p), self.count * (cpad + spad) + align)
            if st != 0:
                raise RuntimeError("hipMalloc failed (%d)" % st)
            self._hip_ptr = p.value
            base = -(-p.value // align) * align
        ts = torch.empty(2, dtype=torch.float32, device="cuda")
        gen = torch.Generator(device="cuda")
        for c in range(self.count):
            gen.manual_seed(seed + c)
            W = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
            if zero_outlier:
                zero_outlier_(torch, W, gen)
            if alloc == "torch":
                self.copies.append(nv.PackedWeight.from_float(W))
            else:
                cp = base + c * (cpad + spad)
                sp = cp + cpad
                st = nv.lib().nvfp4_quantize_packed(W.data_ptr(), 0, N, K, cp, sp, ts.data_ptr(),
                                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if st != 0:
                    raise RuntimeError("nvfp4_quantize_packed failed (%d)" % st)
                self.copies.append(nv.PackedWeight(_RawBuf(cp), _RawBuf(sp), float(ts[0].item()), N, K))
            del W
        torch.cuda.synchronize()

    def release(self, torch):
        torch.cuda.synchronize()
        self.copies = []
        self._slab = None
        if self._hip_ptr is not None:
            hip().hipFree(ctypes.c_void_p(self._hip_ptr))
            self._hip_ptr = None


def make_x(torch, n, K, seed, row_scale=False):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn((n, K), generator=gen, device="cuda", dtype=torch.float32)
    if row_scale:   # per-token row scale U(0.5, 2)
        x = x * (0.5 + 1.5 * torch.rand((n, 1), generator=gen, device="cuda", dtype=torch.float32))
    return x.to(torch.bfloat16)


def graph_upload(torch, g):
    """Upload an instantiated graph to the device (hipGraphUpload) so its
    first replay does not pay the upload inside a timed region."""
    st = hip().hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
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


def settle(torch, g, seconds=SETTLE_S):
    """Untimed replays until `seconds` of wall time have passed."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        g.replay()
        torch.cuda.synchronize()


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


class Timing:
    """Seconds per call: the mean over every timed replay and the p10 / p50 /
    p90 of the per-replay means."""

    def __init__(self, mean, per_replay):
        self.mean = mean
        self.per = sorted(per_replay)

    def pct(self, q):
        return self.per[min(len(self.per) - 1, int(q * len(self.per)))]


def time_calls(torch, call, count, replays=8):
    """Time per call of call(i) for i cycling over `count` rotation slots: a
    graph of 2*count launches, one untimed replay, then `replays` timed
    replays with an event after each (on the stream the graph runs on)."""
    L = 2 * count
    g = capture(torch, call, L)
    g.replay()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    torch.cuda.synchronize()
    ev[0].record(s)
    for e in ev[1:]:
        g.replay()
        e.record(s)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) * 1e-3 / L for a, b in zip(ev[:-1], ev[1:])]
    mean = ev[0].elapsed_time(ev[-1]) * 1e-3 / (L * replays)
    del g
    return Timing(mean, per)


def point(tm, wb, n, t1=None, warm=None):
    from nvfp4_weight_only_02_amd import metrics
    t = tm.mean
    r = {"us": round(t * 1e6, 3),
         "p10_us": round(tm.pct(0.1) * 1e6, 3), "p50_us": round(tm.pct(0.5) * 1e6, 3),
         "p90_us": round(tm.pct(0.9) * 1e6, 3),
         "weight_GBps": round(wb / t / 1e9, 1),
         "frac_hbm_peak": round(wb / t / 1e9 / metrics.HBM_PEAK_GBPS, 4),
         "gemv_tokens_per_s": round(n / t, 1)}
    if t1:
        r["t_over_t1"] = round(t / t1, 3)
    if warm is not None:
        r["warm_us"] = round(warm.mean * 1e6, 3)
    return r


def sweep_shape(torch, rot, n_list, call, x_seed, row_scale=False, warm=True):
    """Cold (rotation) and warm (same copy) time per call for each n."""
    from nvfp4_weight_only_02_amd import metrics
    wb = metrics.weight_bytes(rot.N, rot.K)
    Xs = make_x(torch, 16, rot.K, x_seed)
    Ys = torch.empty((16, rot.N), dtype=torch.bfloat16, device="cuda")
    gs = capture(torch, lambda i: call(rot.copies[i % rot.count], Xs, Ys), rot.count)
    settle(torch, gs)
    del gs
    out, t1 = {}, None
    for n in n_list:
        X = make_x(torch, n, rot.K, x_seed + n, row_scale)
        Y = torch.empty((n, rot.N), dtype=torch.bfloat16, device="cuda")
        t = time_calls(torch, lambda i: call(rot.copies[i % rot.count], X, Y), rot.count)
        tw = time_calls(torch, lambda i: call(rot.copies[0], X, Y), 32) if warm else None
        if n == 1:
            t1 = t.mean
        out[str(n)] = point(t, wb, n, t1, tw)
    return out


def prefill_sweep(nv, torch, t_gemv16):
    """nvfp4_gemm on the fused QKV weight for n beyond one decode tile: cold
    rotation, time per call, MFMA throughput against the dense bf16 peak, and
    the time ceil(n/16) decode launches of 16 tokens would take (t_gemv16
    each), which is what the decode kernel alone would cost."""
    from nvfp4_weight_only_02_amd import metrics
    N, K = SHAPES["fused_qkv_14336x5120"]
    rp = Rotation(nv, torch, N, K, seed=8100)
    out = {}
    for n in PREFILL_N:
        X = make_x(torch, n, K, 2600 + n)
        Y = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
        if n == PREFILL_N[0]:
            gs = capture(torch, lambda i: nv.gemm(rp.copies[i % rp.count], X, out=Y), rp.count)
            settle(torch, gs)
            del gs
        tm = time_calls(torch, lambda i: nv.gemm(rp.copies[i % rp.count], X, out=Y), rp.count, replays=4)
        t = tm.mean
        tf = metrics.flops(n, N, K) / t / 1e12
        rows, toks, gx, gy = nv.gemm_geometry(n, N, K)
        out[str(n)] = {"us": round(t * 1e6, 3), "p10_us": round(tm.pct(0.1) * 1e6, 3),
                       "p90_us": round(tm.pct(0.9) * 1e6, 3), "TFLOPs": round(tf, 1),
                       "frac_bf16_mfma_peak": round(tf / metrics.BF16_DENSE_TFLOPS, 4),
                       "tokens_per_s": round(n / t, 1),
                       "weight_GBps_once": round(metrics.weight_bytes(N, K) / t / 1e9, 1),
                       "decode_launches_us": round(math.ceil(n / 16) * t_gemv16 * 1e6, 3),
                       "tile": {"rows": rows, "tokens": toks, "grid": [gx, gy]}}
        del X, Y
    rp.release(torch)
    torch.cuda.empty_cache()
    return out


def read_ceiling(torch, N, K):
    """Seconds per read of one weight's bytes with the read-stream probe, over
    a >= 1 GiB rotation of distinct buffers (the same cold regime)."""
    from nvfp4_weight_only_02_amd import metrics, probes
    wb = metrics.weight_bytes(N, K)
    count = max(2, math.ceil(ROTATION_BYTES / wb))
    bufs = [torch.full((wb,), c & 0xFF, dtype=torch.uint8, device="cuda") for c in range(count)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    tm = time_calls(torch, lambda i: probes.read_stream(bufs[i % count], sink), count, replays=6)
    del bufs
    torch.cuda.empty_cache()
    t = tm.mean
    return {"us": round(t * 1e6, 3), "p10_us": round(tm.pct(0.1) * 1e6, 3), "p90_us": round(tm.pct(0.9) * 1e6, 3),
            "GBps": round(wb / t / 1e9, 1), "frac_hbm_peak": round(wb / t / 1e9 / metrics.HBM_PEAK_GBPS, 4)}


def launch_ramp(torch, shapes):
    """What a launch costs besides streaming: the time of an empty launch of
    the GEMV's workgroup count in a graph of back-to-back launches, the rate
    of one 1 GiB read (the streaming rate with the ramp amortised), and for
    each shape the read of its bytes split into streaming at that rate plus a
    fixed remainder."""
    from nvfp4_weight_only_02_amd import metrics, probes
    out = {}
    for wg in (160, 224, 256):
        tm = time_calls(torch, lambda i: probes.empty(wg), 32, replays=8)
        out["empty_launch_us_%dwg" % wg] = round(tm.mean * 1e6, 3)
    big = 1 << 30
    bufs = [torch.full((big,), c, dtype=torch.uint8, device="cuda") for c in range(2)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    tm = time_calls(torch, lambda i: probes.read_stream(bufs[i % 2], sink), 2, replays=6)
    del bufs
    torch.cuda.empty_cache()
    rate = big / tm.mean
    out["read_1GiB_us"] = round(tm.mean * 1e6, 2)
    out["read_1GiB_GBps"] = round(rate / 1e9, 1)
    out["read_1GiB_frac_hbm_peak"] = round(rate / 1e9 / metrics.HBM_PEAK_GBPS, 4)
    for name, (N, K) in shapes.items():
        rc = read_ceiling(torch, N, K)
        wb = metrics.weight_bytes(N, K)
        stream_us = wb / rate * 1e6
        out[name] = {"read_us": rc["us"], "read_frac_hbm_peak": rc["frac_hbm_peak"],
                     "streaming_us_at_1GiB_rate": round(stream_us, 3),
                     "fixed_us": round(rc["us"] - stream_us, 3)}
    return out


def decode_step(nv, torch, n=16):
    """48 distinct ssm_qkvz + 16 distinct fused-QKV matrices in the layer
    order of a 64-layer hybrid model (every 4th layer full attention), one
    projection each per decode step, back to back on one stream."""
    from nvfp4_weight_only_02_amd import metrics
    Nz, Kz = SHAPES["ssm_qkvz_16384x5120"]
    Nq, Kq = SHAPES["fused_qkv_14336x5120"]
    rz = Rotation(nv, torch, Nz, Kz, seed=5100, count=48)
    rq = Rotation(nv, torch, Nq, Kq, seed=6100, count=16)
    X = make_x(torch, n, Kz, 2300 + n)
    Yz = torch.empty((n, Nz), dtype=torch.bfloat16, device="cuda")
    Yq = torch.empty((n, Nq), dtype=torch.bfloat16, device="cuda")
    order = []
    for layer in range(64):
        if layer % 4 == 3:
            order.append(("q", len([o for o in order if o[0] == "q"])))
        else:
            order.append(("z", len([o for o in order if o[0] == "z"])))

    def call(i):
        kind, j = order[i]
        if kind == "q":
            nv.gemv_qkv(rq.copies[j], X, QKV_ROWS, QKV_OFFS, Nq, out=Yq)
        else:
            nv.gemv(rz.copies[j], X, out=Yz)
    g = capture(torch, call, 64)
    settle(torch, g)
    t = time_graph(torch, g, 20) / 20
    total = 48 * metrics.weight_bytes(Nz, Kz) + 16 * metrics.weight_bytes(Nq, Kq)
    del g
    rz.release(torch)
    rq.release(torch)
    torch.cuda.empty_cache()
    return {"n": n, "matrices": "48 ssm_qkvz 16384x5120 + 16 fused QKV 14336x5120",
            "weight_bytes": total, "us_per_step": round(t * 1e6, 2),
            "weight_GBps": round(total / t / 1e9, 1),
            "frac_hbm_peak": round(total / t / 1e9 / metrics.HBM_PEAK_GBPS, 4),
            "timing": "20 replays of a HIP graph of the 64 launches of one step"}


def x_staging(torch, K=5120, ns=(1, 16), reps=16):
    """The GEMV's activation staging alone (nvfp4_probe_x_stage) at the
    headline's K on 256 workgroups of 8 waves, X resident in L2 after the
    first repetition: the loads alone and with the LDS round trip into the
    MFMA layout, per staging on every compute unit (the empty launch taken
    off), and the L2-to-compute-unit rate per XCD the loads imply (32 compute
    units per XCD, each reading all of X)."""
    from nvfp4_weight_only_02_amd import probes
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    empty = time_calls(torch, lambda i: probes.empty(256), 32, replays=8).mean
    out = {"K": K, "workgroups": 256, "stagings_per_launch": reps, "empty_launch_us": round(empty * 1e6, 3)}
    for n in ns:
        X = make_x(torch, n, K, 2600 + n)
        row = {"bytes_per_cu": n * K * 2}
        for name, mode in (("loads", probes.XSTAGE_LOADS), ("full", probes.XSTAGE_FULL)):
            tm = time_calls(torch, lambda i: probes.x_stage(X, 256, reps, mode, sink), 16, replays=6)
            row[name + "_us"] = round((tm.mean - empty) / reps * 1e6, 3)
        row["l2_TBps_per_xcd_loads"] = round(32 * row["bytes_per_cu"] / (row["loads_us"] * 1e-6) / 1e12, 2)
        out["n%d" % n] = row
    return out


def arith_rate(torch, blocks=8192, reps=5):
    """Per-block arithmetic rate of the MFMA and VALU forms (probe library,
    register data on every SIMD, two waves each), and what it implies for the
    fused QKV at one launch: each SIMD runs two waves of 4 row groups x 5 tiles
    x 8 blocks = 160 blocks each."""
    from nvfp4_weight_only_02_amd import probes
    sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    out = {}
    for name, path in (("mfma", probes.RATE_MFMA), ("valu", probes.RATE_VALU)):
        out[name] = {}
        for n in (1, 4, 8, 16):
            probes.block_rate(path, n, blocks, sink)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                probes.block_rate(path, n, blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / reps
            ns = t / blocks * 1e9
            out[name][str(n)] = {"ns_per_block_two_waves_per_simd": round(ns, 3),
                                 "fused_qkv_compute_only_us": round(160 * ns * 1e-3, 3)}
    out["what"] = ("time of one 16-element block of a 16-row group on every SIMD, two waves at once, "
                   "arithmetic only (no loads); fused QKV needs 160 such blocks per SIMD per launch")
    return out


def cpu_baseline(N, K, n, seconds, row_scale):
    """The oracle (fp64, OpenMP over rows) on the headline workload's shape:
    the whole N x K weight for n tokens, repeated until `seconds` of CPU time."""
    import numpy as np
    import oracle as O
    from nvfp4_weight_only_02_amd import inputs, metrics
    W = inputs.weights_f32(N, K, inputs.weight_seed(1))
    codes, scales, g = O.quantize(W)
    X = inputs.activations_bf16(n, K, inputs.act_seed(1, n), row_scale=row_scale)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        O.gemv(codes, scales, g, X)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= seconds and len(times) >= 2:
            break
    t = float(np.median(times))
    cores = O.num_threads()
    # The same call on one thread: a warm-up and the median of 3.
    t1s = []
    for _ in range(4):
        t0 = time.perf_counter()
        O.gemv(codes, scales, g, X, nthreads=1)
        t1s.append(time.perf_counter() - t0)
    t1 = float(np.median(t1s[1:]))
    # One token on all threads: a warm-up and the median of 5.
    X1 = inputs.activations_bf16(1, K, inputs.act_seed(1, 1), row_scale=row_scale)
    tn1 = []
    for _ in range(6):
        t0 = time.perf_counter()
        O.gemv(codes, scales, g, X1)
        tn1.append(time.perf_counter() - t0)
    tn1 = float(np.median(tn1[1:]))
    wb = metrics.weight_bytes(N, K)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(wb / t / 1e9, 4),
        "unit": "effective weight GB/s",
        "gemv_tokens_per_s": round(n / t, 2),
        "cores": cores,
        "kind": "oracle",
        "sample": "full %dx%d NVFP4 weight, n=%d tokens, %d runs, median %.3f s per call"
                  % (N, K, n, len(times), t),
        "single_thread": {"value": round(wb / t1 / 1e9, 4), "gemv_tokens_per_s": round(n / t1, 2),
                          "sample": "same call, median of 3 after a warm-up, %.3f s per call" % t1},
        "n1": {"value": round(wb / tn1 / 1e9, 4), "gemv_tokens_per_s": round(1 / tn1, 2),
               "sample": "one token, all threads, median of 5 after a warm-up, %.4f s per call" % tn1},
        "host": {"cpu_model": cpu_model, "os_cpu_count": os.cpu_count()},
    }


def annotate_counter_bandwidth(sweep: dict, workload: str) -> None:
    """Add the HBM bandwidth rocprofv3's FETCH_SIZE + WRITE_SIZE imply (bytes
    per launch from the committed per-n counter summary / time per call) to
    the sweep points it covers, while that summary matches the kernel code
    and the workload."""
    from nvfp4_weight_only_02_amd import metrics
    try:
        with open(per_n_counters_file(workload)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return
    code = kernel_code_hash()
    if code is None or c.get("kernel_code_sha256_16") != code or c.get("workload") != workload:
        return
    for n, b in c.get("hbm_bytes_per_launch", {}).items():
        if n in sweep:
            gbps = b / (sweep[n]["us"] * 1e-6) / 1e9
            sweep[n]["hbm_GBps_counters"] = round(gbps, 1)
            sweep[n]["frac_hbm_peak_counters"] = round(gbps / metrics.HBM_PEAK_GBPS, 4)


def stored_traffic(workload: str, n: int):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None if the summary is absent, covers another workload or was taken on
    different kernel code."""
    try:
        with open(counters_file(workload, n)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    code = kernel_code_hash()
    if code is None or c.get("kernel_code_sha256_16") != code or c.get("workload") != "%s n=%d" % (workload, n):
        return None
    return c.get("hbm_bytes_per_launch")


def targets(sweeps: dict, decode: dict = None) -> dict:
    """Fraction of HBM peak in effective weight bandwidth at n = 1 and n = 16 on
    each target shape, beside the bar, and the decode-step sweep."""
    out = {"bar": TARGET_BAR}
    for name in TARGET_SHAPES:
        sw = sweeps.get(name)
        if sw and "1" in sw and "16" in sw:
            out[name] = {"n1": sw["1"]["frac_hbm_peak"], "n16": sw["16"]["frac_hbm_peak"],
                         "us": [sw["1"]["us"], sw["16"]["us"]]}
    if decode:
        out["decode_step"] = {"us": decode["us_per_step"], "frac_hbm_peak": decode["frac_hbm_peak"]}
    return out


def summarize(result: dict) -> dict:
    """The compact last line: the headline and what the metric needs, never
    the sweeps themselves (those are in the detail line before it)."""
    keep = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "scaling", "vs_baseline", "dtype", "data", "config", "frac_hbm_peak", "gemv_tokens_per_s",
            "per_call_us_over_replays", "roofline", "frac_read_ceiling")
    s = {k: result[k] for k in keep if k in result}
    cb = result.get("cpu_baseline")
    if cb:
        s["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        s["cpu_baseline"]["gemv_tokens_per_s"] = cb["gemv_tokens_per_s"]
    if "targets" in result:
        s["targets"] = result["targets"]
    ramp = result.get("launch_ramp")
    if ramp:
        s["launch_ramp"] = {k: ramp[k] for k in ramp if not isinstance(ramp[k], dict)}
    s["detail"] = "the bench_detail line before this one (and --detail-out)"
    return s


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--n", type=int, default=16)
    ap.add_argument("--workload", default="ssm_qkvz_16384x5120", choices=sorted(SHAPES))
    ap.add_argument("--sweep", default=",".join(str(v) for v in range(1, 17)),
                    help="token counts of the per-n sweeps ('' = none)")
    ap.add_argument("--detail-out", default=None, help="also write the full results (JSON) to this file")
    ap.add_argument("--prefill-only", action="store_true",
                    help="headline timing, then only the prefill GEMM sweep (for profiling it)")
    ap.add_argument("--quick", action="store_true",
                    help="headline and its per-n sweep only (no other shapes, schedules, decode step)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="only the timed region (for rocprofv3 runs): no sweep, no CPU baseline")
    ap.add_argument("--alloc", default="torch", choices=("torch", "slab", "hip"),
                    help="how the headline's rotation copies are allocated")
    ap.add_argument("--alloc-ab", action="store_true",
                    help="time the headline with each allocation of the rotation copies, then exit")
    ap.add_argument("--arith-only", action="store_true",
                    help="run only the MFMA-vs-VALU arithmetic-rate probe and exit")
    ap.add_argument("--x-stage-only", action="store_true",
                    help="run only the activation-staging probe and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_weight_only_02_amd as nv
    from nvfp4_weight_only_02_amd import metrics

    if not (os.path.exists(nv.LIB_PATH) and os.path.exists(os.path.join(ROOT, "nvfp4_weight_only_02_amd",
                                                                        "libnvfp4_probes.so"))):
        from nvfp4_weight_only_02_amd import build as b
        b.build()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch)), flush=True)
        return
    if args.arith_only:
        print(json.dumps({"arith_rate": arith_rate(torch)}), flush=True)
        return
    if args.x_stage_only:
        print(json.dumps({"x_staging": x_staging(torch)}), flush=True)
        return
    N, K = SHAPES[args.workload]
    n = args.n
    qkv = args.workload.startswith("fused_qkv")
    row_scale = args.workload.startswith("ssm_qkvz")

    # Long-K shapes run in K parts (nvfp4_gemv_ws, workspace allocated once,
    # outside the captured graphs); the others in one launch.
    ks = 1 if qkv else nv.gemv_kparts(N, K)
    if qkv:
        def call(w, X, Y):
            nv.gemv_qkv(w, X, QKV_ROWS, QKV_OFFS, N, out=Y)
    elif ks > 1:
        ws = torch.empty(nv.gemv_workspace_bytes(16, N, K, ks), dtype=torch.uint8, device="cuda")

        def call(w, X, Y):
            nv.gemv_ws(w, X, ks, ws, out=Y)
    else:
        def call(w, X, Y):
            nv.gemv(w, X, out=Y)

    X = make_x(torch, n, K, 2000 + n, row_scale)
    Y = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")

    if args.alloc_ab:
        ab = {}
        for mode in ("torch", "slab", "hip", "torch"):
            r = Rotation(nv, torch, N, K, seed=1100, alloc=mode)
            gs = capture(torch, lambda i: call(r.copies[i % r.count], X, Y), r.count)
            settle(torch, gs)
            del gs
            tm = time_calls(torch, lambda i: call(r.copies[i % r.count], X, Y), r.count, replays=40)
            ab.setdefault(mode, []).append({"us": round(tm.mean * 1e6, 3), "p10_us": round(tm.pct(0.1) * 1e6, 3),
                                            "p90_us": round(tm.pct(0.9) * 1e6, 3)})
            r.release(torch)
            torch.cuda.empty_cache()
            log("alloc", mode, ab[mode][-1])
        print(json.dumps({"alloc_ab": {"workload": args.workload, "n": n, "per_mode": ab}}), flush=True)
        return

    log("building rotation of %s copies (%s) ..." % (args.workload, args.alloc))
    rot = Rotation(nv, torch, N, K, seed=1100, alloc=args.alloc)
    log("rotation: %d copies, %.2f GiB" % (rot.count, rot.count * metrics.weight_bytes(N, K) / 2**30))

    # The K timed steps replay one graph of L launches K/L times (L the
    # largest divisor of K up to 64; very long graphs add per-node overhead).
    L = max(d for d in range(1, min(args.steps, 64) + 1) if args.steps % d == 0)
    gt = capture(torch, lambda i: call(rot.copies[i % rot.count], X, Y), L)
    settle(torch, gt)
    # Warm-up: W steps, as whole replays of the timed graph plus a remainder graph.
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
    # Spread of the per-call time across replays: a second pass of the same
    # replays with an event after each, outside the timed region.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps // L + 1)]
    marks[0].record(s)
    for ev in marks[1:]:
        gt.replay()
        ev.record(s)
    torch.cuda.synchronize()
    per_replay = Timing(t_call, [a.elapsed_time(b) * 1e-3 / L for a, b in zip(marks[:-1], marks[1:])])

    wb = metrics.weight_bytes(N, K)
    ab = metrics.algorithmic_bytes(n, N, K)
    value = wb / t_call / 1e9
    wg, waves, tpw = nv.launch_geometry(n, N, K)
    mt, nvq, exact, kc, kparts = nv.gemv_variant(n, N, K, 1 if qkv else 0)
    kernel = "nvfp4_gemv_kernel<%d, %d, %s, %s, %s>" % (mt, nvq, "true" if exact else "false",
                                                        "true" if kc > 1 else "false",
                                                        "true" if kparts > 1 else "false")
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "value_is": "effective weight GB/s at the headline n: NVFP4 weight bytes N*K*9/16 per call / time per call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_call * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "arithmetic": "bf16 MFMA operands (NVFP4 weights decoded exactly: e2m1 codes to bf16, e4m3 block "
                      "scale applied with fp32 FMAs), fp32 accumulation, bf16 output",
        "data": "synthetic: W ~ N(0,0.02) fp32 quantised on the GPU, x ~ N(0,1) bf16%s; %d distinct weight "
                "copies rotated (%.2f GiB, cold against the 256 MB Infinity Cache)"
                % (" x U(0.5,2) per token row" if row_scale else "", rot.count, rot.count * wb / 2**30),
        "config": {"workload": args.workload, "N": N, "K": K, "n_tokens": n,
                   "entry": "nvfp4_gemv_qkv" if qkv else ("nvfp4_gemv_ws" if ks > 1 else "nvfp4_gemv"),
                   "launch": ({"workgroups": wg, "waves_per_workgroup": waves, "tiles_per_wave": tpw}
                              if ks == 1 else {"k_parts": ks}),
                   "rotation_alloc": args.alloc,
                   "timing": "%d replays of a HIP graph of %d launches, HIP events on the launch stream"
                             % (args.steps // L, L)},
        "frac_hbm_peak": round(value / metrics.HBM_PEAK_GBPS, 4),
        "gemv_tokens_per_s": round(n / t_call, 1),
        "host_wall_s_timed_region": round(t_host, 6),
        "per_call_us_over_replays": {"p10": round(per_replay.pct(0.1) * 1e6, 3),
                                     "p50": round(per_replay.pct(0.5) * 1e6, 3),
                                     "p90": round(per_replay.pct(0.9) * 1e6, 3),
                                     "replays": len(per_replay.per), "launches_per_replay": L},
        "roofline": {
            "bound": "hbm",
            "achieved": round(ab / t_call / 1e9, 1),
            "peak": metrics.HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(ab / t_call / 1e9 / metrics.HBM_PEAK_GBPS, 4),
            "traffic": stored_traffic(args.workload, n),
            "kernel": kernel if ks == 1 else kernel + " + nvfp4_ksplit_reduce_kernel",
            "algorithmic_bytes_per_launch": ab,
        },
        "context_pages": PAGES_CONTEXT,
    }
    del gt
    if args.profile_only:
        print(json.dumps(summarize(result)), flush=True)
        return
    if args.prefill_only:
        rot.release(torch)
        torch.cuda.empty_cache()
        result["prefill_fused_qkv"] = prefill_sweep(nv, torch, t_call)
        print(json.dumps({"bench_detail": result}), flush=True)
        print(json.dumps(summarize(result)), flush=True)
        return

    n_list = [int(v) for v in args.sweep.split(",") if v.strip()]
    sweeps = {}
    plain = lambda w, X_, Y_: nv.gemv(w, X_, out=Y_)
    if n_list:
        log("per-n sweep %s ..." % args.workload)
        sweeps[args.workload] = sweep_shape(torch, rot, n_list, call, 2000, row_scale=row_scale)
        annotate_counter_bandwidth(sweeps[args.workload], args.workload)
        if qkv:
            sweeps[args.workload + " (plain nvfp4_gemv)"] = sweep_shape(torch, rot, n_list, plain, 2000, warm=False)
    if args.workload.startswith("ssm_qkvz") and not args.quick:
        log("ssm_qkvz schedules ...")
        sched = {}
        for nn in (n_list or [16]):
            Xs = make_x(torch, nn, K, 2300 + nn, row_scale=True)
            Ys = torch.empty((nn, N), dtype=torch.bfloat16, device="cuda")
            greedy = nv.schedule_greedy(nn, 3)
            row = {"greedy_3": greedy,
                   "greedy_us": round(time_calls(torch, lambda i: nv.gemv_sched(
                       rot.copies[i % rot.count], Xs, greedy, out=Ys), rot.count, replays=4).mean * 1e6, 3),
                   "one_launch_us": sweeps.get(args.workload, {}).get(str(nn), {}).get("us")}
            if nn == 16:
                for name, w in (("8+8", [8, 8]), ("4x4", [4, 4, 4, 4]), ("16", [16])):
                    row[name + "_us"] = round(time_calls(torch, lambda i: nv.gemv_sched(
                        rot.copies[i % rot.count], Xs, w, out=Ys), rot.count, replays=4).mean * 1e6, 3)
            sched[str(nn)] = row
        result["schedules_ssm_qkvz"] = sched
    rot.release(torch)
    del rot
    torch.cuda.empty_cache()

    if not args.quick:
        for name, seed, xs in (("fused_qkv_14336x5120", 3600, 2200), ("ssm_qkvz_16384x5120", 3100, 2300),
                               ("ssm_out_proj_5120x6144", 4100, 2400)):
            if name == args.workload or not n_list:
                continue
            log("%s: sweep ..." % name)
            Ns, Ks = SHAPES[name]
            r = Rotation(nv, torch, Ns, Ks, seed=seed)
            if name.startswith("fused_qkv"):
                qcall = lambda w, X_, Y_: nv.gemv_qkv(w, X_, QKV_ROWS, QKV_OFFS, Ns, out=Y_)
                sweeps[name] = sweep_shape(torch, r, n_list, qcall, xs)
                sweeps[name + " (plain nvfp4_gemv)"] = sweep_shape(torch, r, n_list, plain, xs, warm=False)
            else:
                sweeps[name] = sweep_shape(torch, r, n_list, plain, xs, row_scale=name.startswith("ssm_qkvz"))
            annotate_counter_bandwidth(sweeps[name], name)
            r.release(torch)
            torch.cuda.empty_cache()
        No, Ko = SHAPES["ssm_out_proj_5120x6144"]
        log("ssm_out_proj: zero/outlier tensor ...")
        rzo = Rotation(nv, torch, No, Ko, seed=4600, zero_outlier=True)
        sweeps["ssm_out_proj_5120x6144 (1% zero + 1% outlier blocks)"] = sweep_shape(
            torch, rzo, [1, 4, 16], plain, 2400, warm=False)
        rzo.release(torch)
        torch.cuda.empty_cache()

        log("launch ramp and read ceilings ...")
        result["launch_ramp"] = launch_ramp(torch, {k: SHAPES[k] for k in TARGET_SHAPES})
        rc = result["launch_ramp"][args.workload] if args.workload in result["launch_ramp"] else None
        if rc:
            result["frac_read_ceiling"] = round(rc["read_us"] * 1e-6 / t_call, 4)

        log("decode-step sweep ...")
        result["decode_step"] = decode_step(nv, torch)

        extra = {}
        for name, Ne, Ke, rows, what in EXTRA_SHAPES:
            log("extra shape %s ..." % name)
            re_ = Rotation(nv, torch, Ne, Ke, seed=7100 + Ne % 997)
            if rows:
                offs = (0, rows[0], rows[0] + rows[1])
                ecall = (lambda rws, ofs, ld: lambda w, X_, Y_: nv.gemv_qkv(w, X_, rws, ofs, ld, out=Y_))(rows, offs, Ne)
            else:
                ecall = plain
            wg_, wv_, tpw_ = nv.launch_geometry(16, Ne, Ke)
            extra[name] = {"what": what, "N": Ne, "K": Ke,
                           "launch": {"workgroups": wg_, "tiles_per_wave": tpw_},
                           "sweep": sweep_shape(torch, re_, EXTRA_N, ecall, 2500, warm=False),
                           "read_ceiling": read_ceiling(torch, Ne, Ke)}
            kse = nv.gemv_kparts(Ne, Ke)
            if kse > 1 and not rows:
                # K parts: partials in a workspace allocated once, outside the
                # captured graphs, then the fixed-order reduction launch.
                wse = torch.empty(nv.gemv_workspace_bytes(max(EXTRA_N), Ne, Ke, kse), dtype=torch.uint8,
                                  device="cuda")
                kcall = (lambda k_, ws_: lambda w, X_, Y_: nv.gemv_ws(w, X_, k_, ws_, out=Y_))(kse, wse)
                extra[name]["k_parts"] = {"ks": kse, "entry": "nvfp4_gemv_ws",
                                          "sweep": sweep_shape(torch, re_, EXTRA_N, kcall, 2500, warm=False)}
                del wse
            re_.release(torch)
            torch.cuda.empty_cache()
        result["extra_shapes"] = extra

        log("MFMA vs VALU arithmetic rate ...")
        result["arith_rate"] = arith_rate(torch)
        log("activation staging probe ...")
        result["x_staging"] = x_staging(torch)

        log("prefill GEMM sweep ...")
        result["prefill_fused_qkv"] = prefill_sweep(nv, torch, t_call)

    result["sweep"] = sweeps
    result["targets"] = targets(sweeps, result.get("decode_step"))
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        result["cpu_baseline"] = cpu_baseline(N, K, n, args.cpu_seconds, row_scale)

    detail = json.dumps({"bench_detail": result})
    if args.detail_out:
        with open(args.detail_out, "w") as f:
            f.write(detail + "\n")
    print(detail, flush=True)
    print(json.dumps(summarize(result)), flush=True)


if __name__ == "__main__":
    main()
