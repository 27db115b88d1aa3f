"""Edge cases of every compute entry point against the CPU oracle, through the
C ABI: the longest K the library takes (262144 columns, 37 K-chunk passes in
one GEMV launch), many row groups per workgroup (several batches of LDS
partial slots), the largest token count of one GEMM call, and block scales
that quantise to E4M3 subnormals and zero.  Same bar as the other GEMV tests:
|y - y_ref| <= 1e-3 * sum_k |w x| + one bf16 ulp of y_ref, y_ref the oracle's
fp64 sum; token identity across n is bit-exact.
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


def packed(W):
    codes, scales, g = O.quantize(W)
    N, K = W.shape
    pw = nv.PackedWeight.from_canonical(to_dev_u8(codes), to_dev_u8(scales), g, N, K)
    return pw, codes, scales, g


@pytest.fixture(scope="module")
def longest_k():
    N, K = 40, 1 << 18
    say("build %dx%d" % (N, K))
    pw, codes, scales, g = packed(inputs.weights_f32(N, K, 8800))
    X = inputs.activations_bf16(40, K, 8801)
    Yref, Aref = O.gemv(codes, scales, g, X)
    return pw, X, Yref, Aref


def test_gemv_longest_k(longest_k):
    say("gemv at K = 262144 (37 K-chunk passes)")
    pw, X, Yref, Aref = longest_k
    Xd = x_to_dev(X[:16])
    full = y_bits(nv.gemv(pw, Xd))
    assert_parity(full, Yref[:16], Aref[:16], "gemv 40x262144 n=16")
    for n in (1, 7):
        assert np.array_equal(y_bits(nv.gemv(pw, Xd[:n].contiguous())), full[:n]), n


def test_gemm_longest_k(longest_k):
    say("gemm at K = 262144")
    pw, X, Yref, Aref = longest_k
    assert_parity(y_bits(nv.gemm(pw, x_to_dev(X))), Yref, Aref, "gemm 40x262144 n=40")


def test_many_row_groups_per_workgroup():
    """131072 rows: 8192 row groups, 32 per workgroup, so the LDS partial
    slots (8 row groups) are filled and reduced four times per launch."""
    N, K = 131072, 256
    say("gemv %dx%d, 32 row groups per workgroup" % (N, K))
    pw, codes, scales, g = packed(inputs.weights_f32(N, K, 8900))
    wg, _, _ = nv.launch_geometry(16, N, K)
    assert -(-(N // 16) // wg) == 32
    X = inputs.activations_bf16(16, K, 8901)
    Yref, Aref = O.gemv(codes, scales, g, X)
    Xd = x_to_dev(X)
    full = y_bits(nv.gemv(pw, Xd))
    assert_parity(full, Yref, Aref, "gemv %dx%d n=16" % (N, K))
    assert np.array_equal(y_bits(nv.gemv(pw, Xd[:3].contiguous())), full[:3])


def test_gemm_largest_token_count():
    n = 1 << 20      # the largest n of one nvfp4_gemm call
    N, K = 17, 32
    say("gemm with n = %d" % n)
    pw, codes, scales, g = packed(inputs.weights_f32(N, K, 9000))
    X = inputs.activations_bf16(n, K, 9001)
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(y_bits(nv.gemm(pw, x_to_dev(X))), Yref, Aref, "gemm %dx%d n=%d" % (N, K, n))


def test_subnormal_and_zero_block_scales():
    """Blocks scaled over 2^0 .. 2^-26 before quantisation: their E4M3 scales
    land on normals, subnormals (0x01..0x07) and zero."""
    N, K = 300, 9216
    say("subnormal and zero block scales %dx%d" % (N, K))
    rng = np.random.default_rng(77)
    W = inputs.weights_f32(N, K, 7700)
    mult = np.exp2(-rng.uniform(0, 26, size=(N, K // 16))).astype(np.float32)
    W = (W.reshape(N, K // 16, 16) * mult[:, :, None]).reshape(N, K)
    pw, codes, scales, g = packed(W)
    s = scales.ravel()
    assert (s == 0).any() and ((s > 0) & (s < 8)).any() and (s == 0x7E).any()
    X = inputs.activations_bf16(40, K, 7701)
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(y_bits(nv.gemv(pw, x_to_dev(X[:16]))), Yref[:16], Aref[:16], "gemv")
    assert_parity(y_bits(nv.gemv_ws(pw, x_to_dev(X[:16]))), Yref[:16], Aref[:16], "gemv_ws")
    assert_parity(y_bits(nv.gemm(pw, x_to_dev(X))), Yref, Aref, "gemm")


def test_very_many_rows():
    """N = 2^24 + 5 rows (1048577 row groups, about 4096 per workgroup, the last
    one ragged) at K = 128: row, row-group and output offsets beyond 2^24,
    checked on the first and last rows and a stride through the rest, and the
    first token against the same token alone."""
    N, K, n = (1 << 24) + 5, 128, 3
    say("gemv %dx%d n=%d" % (N, K, n))
    rng = np.random.default_rng(9100)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x28, 0x48, size=(N, K // 16), dtype=np.uint8)
    g = 1.0 / 256
    pw = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                        g, N, K)
    X = inputs.activations_bf16(n, K, 9101)
    Xd = x_to_dev(X)
    full = y_bits(nv.gemv(pw, Xd))
    rows = np.array(sorted(set(list(range(0, 64)) + list(range(N - 64, N)) + list(range(0, N, 65537)))))
    Yref, Aref = O.gemv(np.ascontiguousarray(codes[rows]), np.ascontiguousarray(scales[rows]), g, X)
    assert_parity(full[:, rows], Yref, Aref, "gemv %dx%d n=%d (sampled rows)" % (N, K, n))
    assert np.array_equal(y_bits(nv.gemv(pw, Xd[:1].contiguous()))[0], full[0])
