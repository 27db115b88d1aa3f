"""Non-finite and subnormal inputs on the GPU path, against the oracle's IEEE
fp64 sums.

A decode batch carries unrelated sequences, so a NaN or infinity in one
token's activations must reach that token's outputs only, and a NaN scale
byte (E4M3 0x7F / 0xFF) must reach its own weight row only; every other
output stays bit-identical to the run without the bad value.  Where the bad
value does reach, the outputs take the IEEE categories of the exact sum: an
infinite activation times a zero weight (a zero code or a zero scale) is
NaN, times a non-zero weight an infinity of the product's sign; a NaN
activation or scale gives NaN.  Subnormal bf16 activations are summed like
any other value (no flush to zero).
"""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from nvfp4_weight_only_02_amd import inputs

pytestmark = pytest.mark.gpu

BF16_POS_INF, BF16_NEG_INF, BF16_NAN = 0x7F80, 0xFF80, 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    nv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def x_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def y_bits(Y: torch.Tensor) -> np.ndarray:
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def packed(codes, scales, g, N, K) -> nv.PackedWeight:
    return nv.PackedWeight.from_canonical(torch.from_numpy(np.ascontiguousarray(codes)).cuda(),
                                          torch.from_numpy(np.ascontiguousarray(scales)).cuda(), g, N, K)


def assert_categories(got_bits: np.ndarray, ref: np.ndarray, what: str):
    """The GPU output is NaN exactly where the oracle's is, and the same signed
    infinity wherever the oracle's is infinite."""
    got = O.bf16_bits_to_f64(got_bits)
    nan_ref = np.isnan(ref)
    inf_ref = np.isinf(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "%s: NaN pattern differs (%d vs %d NaNs)" % (
        what, int(np.isnan(got).sum()), int(nan_ref.sum()))
    assert np.array_equal(got[inf_ref], ref[inf_ref]), "%s: infinities differ" % what


def bad_activations(X: np.ndarray, plan, seed: int):
    """X with the planted values: plan is [(token, bf16 bits), ...], each at a
    seeded column."""
    rng = np.random.default_rng(seed)
    Xb = X.copy()
    cols = []
    for t, bits in plan:
        k = int(rng.integers(0, X.shape[1]))
        Xb[t, k] = bits
        cols.append(k)
    return Xb, cols


@pytest.mark.parametrize("N,K,n,path", [
    (1000, 2560, 8, "gemv"),            # ragged rows, K not a multiple of 8 tiles
    (16384, 5120, 16, "gemv"),          # the decode launch of the largest projection
    (600, 17408, 16, "gemv_ws"),        # K parts and the reduction launch
    (900, 1536, 40, "gemm"),            # prefill form, tokens across two token tiles
])
def test_nonfinite_activation_stays_in_its_token(N, K, n, path):
    say("nonfinite activation", N, K, n, path)
    W = inputs.weights_f32(N, K, 4100 + N)
    codes, scales, g = O.quantize(W)
    w = packed(codes, scales, g, N, K)
    X = inputs.activations_bf16(n, K, 4200 + n)
    plan = [(n // 4, BF16_POS_INF), (n // 2, BF16_NEG_INF), (n - 1, BF16_NAN)]
    Xb, cols = bad_activations(X, plan, 4300 + n)
    run = {"gemv": nv.gemv, "gemm": nv.gemm, "gemv_ws": nv.gemv_ws}[path]
    clean = y_bits(run(w, x_to_dev(X)))
    bad = y_bits(run(w, x_to_dev(Xb)))
    torch.cuda.synchronize()
    hit = sorted({t for t, _ in plan})
    others = [t for t in range(n) if t not in hit]
    assert np.array_equal(bad[others], clean[others]), "a planted value leaked into another token"
    # The planted tokens, against the oracle: every row if small, else a sample
    # that covers the first, last and random rows.
    if N <= 2000:
        rows = np.arange(N)
    else:
        rng = np.random.default_rng(4400)
        rows = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.integers(0, N, 96)]))
    ref, _ = O.gemv(codes[rows], scales[rows], g, Xb[hit])
    assert_categories(bad[hit][:, rows], ref, "planted tokens")
    # The infinite activations reach every row: NaN where the weight at their
    # column is zero, an infinity elsewhere (no finite output left).
    assert not np.isfinite(ref).any()
    zero_w = (O.dequant(codes[rows], scales[rows], g)[:, cols[0]] == 0)
    assert zero_w.any() and (~zero_w).any(), "the sample should hold zero and non-zero weights"


@pytest.mark.parametrize("N,K,n", [(1000, 2560, 8), (16384, 5120, 16)])
def test_nan_scale_byte_stays_in_its_row(N, K, n):
    say("nan scale byte", N, K, n)
    W = inputs.weights_f32(N, K, 4500 + N)
    codes, scales, g = O.quantize(W)
    X = inputs.activations_bf16(n, K, 4600 + n)
    rng = np.random.default_rng(4700)
    rows = [int(rng.integers(0, N)), N - 1]
    sb = scales.copy()
    sb[rows[0], int(rng.integers(0, K // 16))] = 0x7F
    sb[rows[1], 0] = 0xFF
    clean = y_bits(nv.gemv(packed(codes, scales, g, N, K), x_to_dev(X)))
    bad = y_bits(nv.gemv(packed(codes, sb, g, N, K), x_to_dev(X)))
    torch.cuda.synchronize()
    keep = np.setdiff1d(np.arange(N), rows)
    assert np.array_equal(bad[:, keep], clean[:, keep]), "a NaN scale leaked into another row"
    ref, _ = O.gemv(codes[rows], sb[rows], g, X)
    assert np.isnan(ref).all()
    assert_categories(bad[:, rows], ref, "rows with a NaN scale")


@pytest.mark.parametrize("N,K,n", [(1000, 2560, 8), (16384, 5120, 16)])
def test_subnormal_activations(N, K, n):
    """bf16 subnormal activations (exponent field 0) take part in the sum like
    any other value: a token whose activations are all subnormal gets the
    oracle's (normal, tiny) result, not the zero a flush would give."""
    say("subnormal activations", N, K, n)
    W = inputs.weights_f32(N, K, 4800 + N)
    codes, scales, g = O.quantize(W)
    rng = np.random.default_rng(4900 + n)
    X = inputs.activations_bf16(n, K, 5000 + n)
    sub = (rng.integers(1, 128, size=K) | (rng.integers(0, 2, size=K) << 15)).astype(np.uint16)
    X[0] = sub                          # token 0: every activation subnormal
    X[n - 1, ::2] = sub[::2]            # last token: half of them
    Y = y_bits(nv.gemv(packed(codes, scales, g, N, K), x_to_dev(X)))
    torch.cuda.synchronize()
    rows = np.arange(N) if N <= 2000 else np.unique(np.concatenate(
        [np.arange(16), np.arange(N - 16, N), np.random.default_rng(5100).integers(0, N, 96)]))
    ref, acc = O.gemv(codes[rows], scales[rows], g, X)
    got = O.bf16_bits_to_f64(Y[:, rows])
    tol = O.tolerance(ref, acc)
    assert (np.abs(ref[0]) > 0).mean() > 0.9, "the all-subnormal token should give non-zero results"
    assert (np.abs(got - ref) <= tol).all(), "worst err/tol %.3g" % float(np.max(np.abs(got - ref) / tol))
