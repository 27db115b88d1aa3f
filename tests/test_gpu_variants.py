"""Every GEMV kernel instantiation the dispatcher can launch, on the GPU, through
the C ABI: one small case per instantiation (tests/kernel_variants.py), each
checked against the CPU oracle on sampled rows and, on every row, for
bit-identity of its first and last tokens with the same token launched alone
(n = 1, a different instantiation).

The weights are random code and scale bytes (parity is defined on the packed
bytes, so any bytes are a valid weight): 8200 rows, so that every workgroup
streams several 16-row groups (the ring refills between them) and the last
row group is ragged.  Scales are E4M3 bytes 0x28 .. 0x47 (2^-2 .. 2^1.9),
gscale 1/128.
"""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from kernel_variants import COVER_N, coverage_cases, kernel_of, variant
from nvfp4_weight_only_02_amd import inputs

pytestmark = pytest.mark.gpu

GSCALE = 1.0 / 128
# Sampled 16-row groups: a stride through all 513, the first workgroup's
# groups and the ragged last one.
SAMPLE_RG = sorted(set(list(range(0, 513, 23)) + [1, 2, 511, 512]))
SAMPLE_ROWS = np.array([r for g in SAMPLE_RG for r in range(16 * g, min(16 * g + 16, COVER_N))])


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    nv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def pool():
    rng = np.random.default_rng(77)
    codes = rng.integers(0, 256, size=(COVER_N, 16384 // 2), dtype=np.uint8)
    scales = rng.integers(0x28, 0x48, size=(COVER_N, 16384 // 16), dtype=np.uint8)
    return codes, scales


def x_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def y_bits(Y):
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def run(pw, X, ks):
    if ks == 1:
        return y_bits(nv.gemv(pw, X))
    return y_bits(nv.gemv_ws(pw, X, ks))


@pytest.mark.parametrize("N,K,n,ks", coverage_cases())
def test_every_kernel_variant(pool, N, K, n, ks):
    v = variant(n, K, ks)
    say("variant", kernel_of(v), "N=%d K=%d n=%d ks=%d" % (N, K, n, ks))
    assert nv.gemv_variant(n, N, K, ks) == v
    codes = np.ascontiguousarray(pool[0][:, :K // 2])
    scales = np.ascontiguousarray(pool[1][:, :K // 16])
    pw = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                        GSCALE, N, K)
    X = inputs.activations_bf16(n, K, 4000 + K + n)
    Xd = x_to_dev(X)
    Y = run(pw, Xd, ks)
    Yref, Aref = O.gemv(np.ascontiguousarray(codes[SAMPLE_ROWS]), np.ascontiguousarray(scales[SAMPLE_ROWS]),
                        GSCALE, X)
    y = O.bf16_bits_to_f64(Y[:, SAMPLE_ROWS])
    tol = O.tolerance(Yref, Aref)
    err = np.abs(y - Yref)
    assert (err <= tol).all(), "%s: %d outside tolerance, worst err/tol %.3g" % (
        kernel_of(v), int((err > tol).sum()), float((err / tol).max()))
    for t in sorted({0, n - 1}):
        one = run(pw, Xd[t:t + 1].contiguous(), ks)
        assert np.array_equal(one[0], Y[t]), (kernel_of(v), t)
