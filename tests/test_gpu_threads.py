"""Several host threads calling the library at once.

ctypes releases the GIL for the duration of a call, so the library's host
side (argument checks, the per-device lookup of compute units and
architecture, launch geometry) runs concurrently here.  Each thread uses its
own stream, weights, activations and workspace, and must get the bits the
same calls give one after another.
"""
import threading

import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from nvfp4_weight_only_02_amd import inputs

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 10


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    nv.lib()
    yield
    torch.cuda.synchronize()


def y_bits(Y: torch.Tensor) -> np.ndarray:
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def case(i):
    """Thread i's weight (a different shape per thread), activations and workspace."""
    N, K = [(3000, 5120), (2048, 6144), (1500, 17408), (4096, 2048)][i]
    codes, scales, g = O.quantize(inputs.weights_f32(N, K, 5200 + i))
    w = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), g, N, K)
    n = [16, 5, 12, 1][i]
    x = torch.from_numpy(inputs.activations_bf16(n, K, 5300 + i).view(np.int16)).cuda().view(torch.bfloat16)
    xg = torch.from_numpy(inputs.activations_bf16(40, K, 5400 + i).view(np.int16)).cuda().view(torch.bfloat16)
    ks = nv.gemv_kparts(N, K) if K > 8192 else 2
    ws = torch.empty(nv.gemv_workspace_bytes(n, N, K, ks), dtype=torch.uint8, device="cuda")
    a, b = N // 2, N // 4
    # q | k | v written in the order v, q, k across the output row
    return dict(w=w, x=x, xg=xg, ks=ks, ws=ws, rows=(a, b, N - a - b), off=(N - a - b, N - b, 0), ldy=N)


def run_all(c):
    return [nv.gemv(c["w"], c["x"]),
            nv.gemv_qkv(c["w"], c["x"], c["rows"], c["off"], c["ldy"]),
            nv.gemv_ws(c["w"], c["x"], c["ks"], workspace=c["ws"]),
            nv.gemm(c["w"], c["xg"])]


def test_host_threads_share_the_library():
    cases = [case(i) for i in range(THREADS)]
    serial = [[y_bits(y) for y in run_all(c)] for c in cases]
    torch.cuda.synchronize()
    start = threading.Barrier(THREADS)
    results, errors = [None] * THREADS, []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(stream):
                start.wait()
                for _ in range(ROUNDS):
                    outs.append(run_all(cases[i]))
            stream.synchronize()
            results[i] = [[y_bits(y) for y in o] for o in outs]
        except Exception as e:   # reported below, in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i in range(THREADS):
        for r, got in enumerate(results[i]):
            for j, (a, b) in enumerate(zip(serial[i], got)):
                assert np.array_equal(a, b), "thread %d round %d call %d differs from the serial bits" % (i, r, j)
