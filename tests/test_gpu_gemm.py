"""GPU parity of the prefill (many-token) GEMM against the CPU oracle, through
the C ABI.

Same definition and bar as the decode GEMV: |y - y_ref| <= 1e-3 * sum_k |w x|
+ one bf16 ulp of y_ref, y_ref the oracle's fp64 sum; bit-exact dequant on
one-hot inputs; bit-identical token results whatever n, the tile shape the
launch picks and the token's place in the batch.  Cases span several token
tiles and row tiles with ragged tails in n, N and K.  The full decode-layer
shape is checked on outputs sampled one by one from the oracle.
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


def packed(codes, scales, g, N, K):
    return nv.PackedWeight.from_canonical(to_dev_u8(codes), to_dev_u8(scales), g, N, K)


def assert_parity(Ybits, Yref, Aref, what=""):
    y = O.bf16_bits_to_f64(Ybits)
    tol = O.tolerance(Yref, Aref)
    err = np.abs(y - Yref)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside tolerance, worst err/tol %.3g" % (
        what, int(bad.sum()), bad.size, float(np.max(err / tol)))


@pytest.mark.parametrize("N,K", [(1, 16), (37, 144), (200, 656), (1024, 1024), (130, 8208)])
@pytest.mark.parametrize("n", [1, 17, 33, 100, 130])
def test_gemm_parity_ragged(N, K, n):
    say("gemm", N, K, n, nv.gemm_geometry(n, N, K))
    W = inputs.weights_f32(N, K, 300 + N + K)
    codes, scales, g = O.quantize(W)
    pw = packed(codes, scales, g, N, K)
    X = inputs.activations_bf16(n, K, 400 + n)
    Y = y_bits(nv.gemm(pw, x_to_dev(X)))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "gemm %dx%d n=%d" % (N, K, n))


def test_gemm_zero_and_outlier_blocks():
    say("gemm zero/outlier 320x6144 n=77")
    N, K, n = 320, 6144, 77
    W = inputs.add_zero_and_outlier_blocks(inputs.weights_f32(N, K, 31), 32)
    codes, scales, g = O.quantize(W)
    X = inputs.activations_bf16(n, K, 33, row_scale=True)
    Y = y_bits(nv.gemm(packed(codes, scales, g, N, K), x_to_dev(X)))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "zero/outlier")


def test_gemm_one_hot_is_exact_dequant():
    """gscale = 1 and token t one-hot at column k0 + t: Y[t][r] = E2M1 * E4M3 exactly."""
    say("gemm one-hot 80x256")
    rng = np.random.default_rng(22)
    N, K = 80, 256
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    pw = packed(codes, scales, 1.0, N, K)
    Wd = O.dequant(codes, scales, 1.0)
    for k0 in (0, 64, 128, 192):
        X = np.zeros((64, K), dtype=np.float32)
        X[np.arange(64), k0 + np.arange(64)] = 1.0
        Y = O.bf16_bits_to_f64(y_bits(nv.gemm(pw, x_to_dev(inputs.f32_to_bf16_bits(X)))))
        assert np.array_equal(Y, Wd[:, k0:k0 + 64].T), k0


def test_gemm_token_identity_across_n_and_tiles():
    """A token's output is the same bits whatever n (hence tile shape: 32-,
    64- and 128-token tiles, 64- and 128-row tiles) and wherever it sits."""
    say("gemm identity 1000x1536")
    N, K = 1000, 1536
    W = inputs.weights_f32(N, K, 41)
    codes, scales, g = O.quantize(W)
    pw = packed(codes, scales, g, N, K)
    X = x_to_dev(inputs.activations_bf16(300, K, 42))
    full = y_bits(nv.gemm(pw, X))
    for a, b in ((0, 1), (5, 6), (0, 17), (0, 64), (100, 164), (37, 300), (250, 300)):
        part = y_bits(nv.gemm(pw, X[a:b].contiguous()))
        assert np.array_equal(part, full[a:b]), (a, b)


def test_gemm_agrees_with_gemv_on_decode_batch():
    """Both entry points meet the bound on the same n <= 16 batch (different
    rounding orders, so not compared bit for bit)."""
    say("gemm vs gemv 512x2048 n=16")
    W = inputs.weights_f32(512, 2048, 51)
    codes, scales, g = O.quantize(W)
    pw = packed(codes, scales, g, 512, 2048)
    X = inputs.activations_bf16(16, 2048, 52)
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(y_bits(nv.gemm(pw, x_to_dev(X))), Yref, Aref, "gemm")
    assert_parity(y_bits(nv.gemv(pw, x_to_dev(X))), Yref, Aref, "gemv")


@pytest.mark.parametrize("n", [256, 320, 1000])
def test_gemm_full_size_sampled(n):
    """Fused QKV 14336 x 5120 at prefill sizes, launched as the bench times
    it; 1500 outputs sampled and computed one by one by the oracle."""
    say("gemm full size fused qkv n", n, nv.gemm_geometry(n, 14336, 5120))
    N, K = 14336, 5120
    W = inputs.weights_f32(N, K, inputs.weight_seed(1))
    codes, scales, g = O.quantize(W)
    pw = packed(codes, scales, g, N, K)
    X = inputs.activations_bf16(n, K, inputs.act_seed(1, n))
    Y = O.bf16_bits_to_f64(y_bits(nv.gemm(pw, x_to_dev(X))))
    rng = np.random.default_rng(n)
    ts = rng.integers(0, n, 1500)
    rs = rng.integers(0, N, 1500)
    ts[:4] = [0, n - 1, 0, n - 1]
    rs[:4] = [0, 0, N - 1, N - 1]
    yref = np.empty(1500)
    aref = np.empty(1500)
    for j, (t, r) in enumerate(zip(ts, rs)):
        yref[j], aref[j] = O.gemv_one(codes, scales, g, X, int(t), int(r))
    err = np.abs(Y[ts, rs] - yref)
    tol = O.tolerance(yref, aref)
    assert (err <= tol).all(), float(np.max(err / tol))


def test_gemm_permutation_negation_scaling():
    """Token permutation permutes rows, negating X negates Y, X * 8 and
    gscale / 4 scale Y exactly (all bit for bit)."""
    say("gemm invariants 700x2048 n=90")
    N, K, n = 700, 2048, 90
    W = inputs.weights_f32(N, K, 61)
    codes, scales, g = O.quantize(W)
    pw = packed(codes, scales, g, N, K)
    X = inputs.activations_bf16(n, K, 62)
    ref = y_bits(nv.gemm(pw, x_to_dev(X)))
    perm = np.random.default_rng(4).permutation(n)
    assert np.array_equal(y_bits(nv.gemm(pw, x_to_dev(X[perm]))), ref[perm])
    assert np.array_equal(y_bits(nv.gemm(pw, x_to_dev(X ^ np.uint16(0x8000)))), ref ^ np.uint16(0x8000))
    X8 = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(X) * np.float32(8))
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(nv.gemm(pw, x_to_dev(X8)))), 8 * O.bf16_bits_to_f64(ref))
    pw4 = nv.PackedWeight(pw.codes, pw.scales, pw.gscale * 0.25, N, K)
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(nv.gemm(pw4, x_to_dev(X)))),
                          0.25 * O.bf16_bits_to_f64(ref))


@pytest.mark.parametrize("n", [17, 200])
def test_gemm_guard_band_untouched(n):
    """Canaries before and after Y stay intact (ragged last row and token tiles)."""
    say("gemm guard band 1000x1024 n", n)
    N, K, G = 1000, 1024, 4096
    W = inputs.weights_f32(N, K, 71)
    codes, scales, g = O.quantize(W)
    pw = packed(codes, scales, g, N, K)
    X = inputs.activations_bf16(n, K, 72)
    buf = torch.full((G + n * N + G,), 3.0, dtype=torch.bfloat16, device="cuda")
    nv.gemm(pw, x_to_dev(X), out=buf[G:G + n * N].view(n, N))
    b = O.bf16_bits_to_f64(y_bits(buf))
    assert (b[:G] == 3.0).all() and (b[G + n * N:] == 3.0).all()
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(y_bits(buf[G:G + n * N].view(n, N)), Yref, Aref, "guard band n=%d" % n)


def test_gemm_identity_across_row_tiles_full_size():
    """Fused QKV weight: n = 40 (64 rows x 64 tokens), 100 (64 x 128, one token
    tile: 8 waves, two per row group), 200 (256 x 64), 320 (256 x 96) and
    1024 (256 x 128) give the same bits for the tokens they share."""
    N, K = 14336, 5120
    shapes = [nv.gemm_geometry(n, N, K)[:2] for n in (40, 100, 200, 320, 1024)]
    say("gemm tiles", shapes)
    assert shapes == [(64, 64), (64, 128), (256, 64), (256, 96), (256, 128)]
    W = inputs.weights_f32(N, K, inputs.weight_seed(1))
    codes, scales, g = O.quantize(W)
    pw = packed(codes, scales, g, N, K)
    X = x_to_dev(inputs.activations_bf16(1024, K, 81))
    big = y_bits(nv.gemm(pw, X))
    for n in (40, 100, 200, 320):
        assert np.array_equal(y_bits(nv.gemm(pw, X[:n].contiguous())), big[:n]), n
