"""The compute entry points inside captured HIP graphs (the way bench.py and a
serving loop run them): every replay, with the program's own eager work and
synchronisations between replays, must give the eager call's bits.  The entry
points record only kernel launches (no memset or copy nodes)."""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from nvfp4_weight_only_02_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    nv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def y_bits(Y):
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def x_dev(n, K, seed):
    bits = inputs.activations_bf16(n, K, seed)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def weight(N, K, seed):
    codes, scales, g = O.quantize(inputs.weights_f32(N, K, seed))
    return nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                          g, N, K)


def replay_equals_eager(fn, out, replays=4, written=None):
    """Capture fn() (which writes `out`, or its columns `written`) in a graph,
    then replay it several times with unrelated eager kernels and a poisoned
    `out` in between: written columns equal the eager call's bits, the others
    keep the poison."""
    cols = np.ones(out.shape[1], dtype=bool) if written is None else written
    out.fill_(float("nan"))
    fn()
    torch.cuda.synchronize()
    eager = y_bits(out).copy()
    poison = eager[:, ~cols].copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    scratch = torch.empty(1 << 20, device="cuda")
    for r in range(replays):
        out.fill_(float("nan"))
        scratch.normal_()                      # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y_bits(out)
        assert np.array_equal(got[:, cols], eager[:, cols]), "replay %d" % r
        assert np.array_equal(got[:, ~cols], poison), "replay %d wrote outside its projections" % r


def test_gemv_in_graph():
    say("gemv graph replays")
    N, K = 5120, 6144
    w = weight(N, K, 7001)
    for n in (1, 16):
        X = x_dev(n, K, 7002 + n)
        Y = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
        replay_equals_eager(lambda: nv.gemv(w, X, out=Y), Y)


def test_gemv_qkv_in_graph():
    say("gemv_qkv graph replays")
    rows, K = (512, 128, 128), 2048
    N = sum(rows)
    w = weight(N, K, 7101)
    X = x_dev(7, K, 7102)
    ldy = N + 40
    Y = torch.empty((7, ldy), dtype=torch.bfloat16, device="cuda")
    written = np.zeros(ldy, dtype=bool)
    written[40:40 + N] = True
    replay_equals_eager(lambda: nv.gemv_qkv(w, X, rows, (40, 40 + 512, 40 + 640), ldy, out=Y), Y,
                        written=written)


def test_gemm_in_graph():
    say("gemm graph replays")
    N, K = 2049, 1040
    w = weight(N, K, 7201)
    for n in (40, 300):
        X = x_dev(n, K, 7202 + n)
        Y = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
        replay_equals_eager(lambda: nv.gemm(w, X, out=Y), Y)


def test_chunked_gemv_in_graph():
    say("chunked gemv graph replays")
    N, K = 300, 17408
    w = weight(N, K, 7301)
    X = x_dev(16, K, 7302)
    Y = torch.empty((16, N), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager(lambda: nv.gemv(w, X, out=Y), Y)


def test_concurrent_streams_give_the_serial_bits():
    """nvfp4_gemv, nvfp4_gemv_ws (each stream with its own workspace) and
    nvfp4_gemm keep no state between calls: launched at the same time on two
    streams (default priority), on different weights and activations, each
    gives the bits it gives alone."""
    wa, wb = weight(5000, 5120, 61), weight(3000, 6144, 62)
    xa, xb = x_dev(16, 5120, 63), x_dev(9, 6144, 64)
    xg = x_dev(40, 5120, 65)
    alone = [y_bits(nv.gemv(wa, xa)), y_bits(nv.gemv(wb, xb)), y_bits(nv.gemv_ws(wa, xa, 4)),
             y_bits(nv.gemv_ws(wb, xb, 3)), y_bits(nv.gemm(wa, xg))]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            y1 = nv.gemv(wa, xa)
            y3 = nv.gemv_ws(wa, xa, 4)
            y5 = nv.gemm(wa, xg)
        with torch.cuda.stream(s2):
            y2 = nv.gemv(wb, xb)
            y4 = nv.gemv_ws(wb, xb, 3)
        torch.cuda.synchronize()
        outs.append([y_bits(y1), y_bits(y2), y_bits(y3), y_bits(y4), y_bits(y5)])
    say("two streams, 3 rounds")
    for got in outs:
        for a, b in zip(alone, got):
            assert np.array_equal(a, b)
