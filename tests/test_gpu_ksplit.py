"""GPU parity of the K-part GEMV (nvfp4_gemv_ws) against the CPU oracle, through
the C ABI.

The operation is the GEMV's, Y = X . dequant(W)^T, with K cut into parts whose
fp32 partials go through a caller-owned workspace and are added in part order
by a second launch.  The bars:
  * |y - y_ref| <= 1e-3 * sum_k |w x| + one bf16 ulp of y_ref (y_ref the
    oracle's fp64 sum), on shapes whose parts end in ragged tiles, whose last
    part is shorter, and at the longest K the library takes;
  * bit-exact: a token's result in an n-token launch equals the n = 1 launch
    at the same part count; ks = 1 equals nvfp4_gemv; the workspace's prior
    contents never reach the output; replays of a captured graph equal the
    eager call.
"""
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


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def y_bits(Y):
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_parity(Ybits, Yref, Aref, what=""):
    y = O.bf16_bits_to_f64(Ybits)
    tol = O.tolerance(Yref, Aref)
    err = np.abs(y - Yref)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside tolerance, worst err/tol %.3g" % (
        what, int(bad.sum()), bad.size, float(np.max(err / tol)))


def case(N, K, seed, zero_outlier=False):
    W = inputs.weights_f32(N, K, seed)
    if zero_outlier:
        W = inputs.add_zero_and_outlier_blocks(W, seed + 7)
    codes, scales, g = O.quantize(W)
    pw = nv.PackedWeight.from_canonical(to_dev_u8(codes), to_dev_u8(scales), g, N, K)
    return pw, codes, scales, g


# (N, K, n, ks): parts of 1..64 tiles, ragged last tiles (K % 128 != 0), a last
# part shorter than the others, ks = 0 (the library's choice) and 1.
RAGGED = [
    (333, 12304, 7, 5),     # 97 tiles: 20+20+20+20+17, last tile 16 columns
    (1000, 9216, 5, 3),     # 72 tiles: 3 x 24
    (2049, 1040, 7, 3),     # 9 tiles: 3 x 3, last tile 16 columns
    (640, 16384, 16, 9),    # 128 tiles: 8 x 15 + 8
    (17, 8208, 3, 0),       # 65 tiles: the library's split of a just-too-long K
    (37, 1152, 2, 3),       # 9 tiles: 3 x 3
    (100, 1280, 16, 4),     # 10 tiles: 3 + 3 + 3 + 1
    (16, 144, 1, 2),        # 2 tiles of 128 and 16 columns
    (1, 16, 1, 1),
    (300, 40000, 12, 0),    # 313 tiles
]


@pytest.mark.parametrize("N,K,n,ks", RAGGED)
def test_ksplit_parity_ragged(N, K, n, ks):
    say("k parts parity", N, K, n, ks)
    pw, codes, scales, g = case(N, K, 9000 + N + K)
    X = inputs.activations_bf16(n, K, 9100 + n)
    Y = y_bits(nv.gemv_ws(pw, x_to_dev(X), ks))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "%dx%d n=%d ks=%d" % (N, K, n, ks))


@pytest.fixture(scope="module")
def ffn_down():
    say("build ffn down 5120x17408")
    N, K = 5120, 17408
    pw, codes, scales, g = case(N, K, inputs.weight_seed(6))
    X = inputs.activations_bf16(16, K, inputs.act_seed(6, 16))
    return pw, codes, scales, g, X


@pytest.mark.parametrize("n", [1, 5, 16])
def test_ksplit_ffn_down_parity(ffn_down, n):
    say("ffn down k parts parity n", n)
    pw, codes, scales, g, X = ffn_down
    assert nv.gemv_kparts(pw.N, pw.K) == 4
    Y = y_bits(nv.gemv_ws(pw, x_to_dev(X[:n])))
    Yref, Aref = O.gemv(codes, scales, g, X[:n])
    assert_parity(Y, Yref, Aref, "ffn down 5120x17408 n=%d, 4 K parts" % n)


def test_ksplit_token_identity(ffn_down):
    say("ffn down k parts identity across n")
    pw, _, _, _, X = ffn_down
    Xd = x_to_dev(X)
    full = y_bits(nv.gemv_ws(pw, Xd))
    for n in range(1, 16):
        assert np.array_equal(y_bits(nv.gemv_ws(pw, Xd[:n].contiguous())), full[:n]), n
    # and on a shape with a short last part and a ragged last tile
    pw2, _, _, _ = case(333, 12304, 9333)
    X2 = x_to_dev(inputs.activations_bf16(16, 12304, 9334))
    full2 = y_bits(nv.gemv_ws(pw2, X2, 5))
    for n in (1, 4, 9, 15):
        assert np.array_equal(y_bits(nv.gemv_ws(pw2, X2[:n].contiguous(), 5)), full2[:n]), n


def test_one_part_equals_gemv(ffn_down):
    say("ks = 1 equals nvfp4_gemv")
    pw, _, _, _, X = ffn_down
    Xd = x_to_dev(X)
    assert np.array_equal(y_bits(nv.gemv_ws(pw, Xd, 1)), y_bits(nv.gemv(pw, Xd)))
    pw2, _, _, _ = case(100, 1280, 9100)
    X2 = x_to_dev(inputs.activations_bf16(5, 1280, 9101))
    assert np.array_equal(y_bits(nv.gemv_ws(pw2, X2, 1)), y_bits(nv.gemv(pw2, X2)))


def test_workspace_contents_never_reach_the_output(ffn_down):
    say("workspace poison, reuse and guard bands")
    pw, _, _, _, X = ffn_down
    Xd = x_to_dev(X)
    clean = y_bits(nv.gemv_ws(pw, Xd))
    need = nv.gemv_workspace_bytes(16, pw.N, pw.K)
    guard = 4096
    ws = torch.full((need + guard,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN floats
    ybuf = torch.full((16 * pw.N + guard,), -1, dtype=torch.int16, device="cuda")
    Y = ybuf[:16 * pw.N].view(torch.bfloat16).view(16, pw.N)
    nv.gemv_ws(pw, Xd, 0, ws, out=Y)
    assert np.array_equal(y_bits(Y), clean)
    # a second, smaller call on the same (now dirty) workspace
    Y3 = ybuf[:3 * pw.N].view(torch.bfloat16).view(3, pw.N)
    nv.gemv_ws(pw, Xd[:3].contiguous(), 0, ws, out=Y3)
    assert np.array_equal(y_bits(Y3), clean[:3])
    torch.cuda.synchronize()
    assert bool((ws[need:] == 0xFF).all()), "workspace written beyond its stated size"
    assert bool((ybuf[16 * pw.N:] == -1).all()), "output written beyond n x N"


def test_ksplit_zero_outlier_blocks():
    say("k parts with zero and outlier blocks")
    N, K = 300, 17408
    pw, codes, scales, g = case(N, K, 9500, zero_outlier=True)
    X = inputs.activations_bf16(16, K, 9501)
    Y = y_bits(nv.gemv_ws(pw, x_to_dev(X)))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "%dx%d zero/outlier n=16" % (N, K))


def test_ksplit_longest_k():
    say("k parts at K = 262144")
    N, K = 40, 1 << 18
    assert nv.gemv_kparts(N, K) == 64
    pw, codes, scales, g = case(N, K, 9600)
    X = inputs.activations_bf16(2, K, 9601)
    Y = y_bits(nv.gemv_ws(pw, x_to_dev(X)))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "%dx%d n=2, 64 K parts" % (N, K))


def test_ksplit_graph_replays_equal_eager(ffn_down):
    say("k parts in a captured graph")
    pw, _, _, _, X = ffn_down
    Xd = x_to_dev(X)
    eager = y_bits(nv.gemv_ws(pw, Xd))
    ws = torch.empty(nv.gemv_workspace_bytes(16, pw.N, pw.K), dtype=torch.uint8, device="cuda")
    Y = torch.empty((16, pw.N), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        nv.gemv_ws(pw, Xd, 0, ws, out=Y)          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.gemv_ws(pw, Xd, 0, ws, out=Y)
    for r in range(3):
        Y.fill_(0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(Y), eager), r


def test_ksplit_full_decode_shape_explicit_parts():
    """ssm_qkvz 16384 x 5120 (one pass, so the library takes one part) cut
    into 2 parts on request: parity at n = 16 against the oracle."""
    say("qkvz 16384x5120 in 2 K parts")
    N, K = 16384, 5120
    pw, codes, scales, g = case(N, K, inputs.weight_seed(3))
    assert nv.gemv_kparts(N, K) == 1
    X = inputs.activations_bf16(16, K, inputs.act_seed(3, 16), row_scale=True)
    Y = y_bits(nv.gemv_ws(pw, x_to_dev(X), 2))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "qkvz 16384x5120 n=16, 2 K parts")


def test_ksplit_identity_every_n():
    say("k parts identity for every n")
    pw, _, _, _ = case(333, 12304, 9444)
    X = x_to_dev(inputs.activations_bf16(16, 12304, 9445))
    full = y_bits(nv.gemv_ws(pw, X, 5))
    for n in range(1, 16):
        assert np.array_equal(y_bits(nv.gemv_ws(pw, X[:n].contiguous(), 5)), full[:n]), n
