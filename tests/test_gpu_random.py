"""Seeded random shapes through every compute entry point, against the CPU
oracle element by element (same bar as the fixed cases: |y - y_ref| <= 1e-3 *
sum_k |w x| + one bf16 ulp of y_ref).  The shapes are drawn so that most of
them are ragged: N not a multiple of 16, K not a multiple of 128 (down to
K = 16), K beyond one 8192-column chunk, odd token counts, and for the fused
QKV entry random projection splits and output offsets; the K-part entry at
the library's part count and at a random valid one."""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from nvfp4_weight_only_02_amd import inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def x_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def y_bits(Y):
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def check(Ybits, Yref, Aref, what):
    y = O.bf16_bits_to_f64(Ybits)
    tol = O.tolerance(Yref, Aref)
    err = np.abs(y - Yref)
    assert (err <= tol).all(), "%s: worst err/tol %.3g" % (what, float(np.max(err / tol)))


def shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        N = int(rng.integers(1, 700))
        kind = rng.integers(0, 4)
        if kind == 0:
            K = 16 * int(rng.integers(1, 9))            # shorter than one tile
        elif kind == 1:
            K = 16 * int(rng.integers(9, 512))          # one chunk, often ragged
        elif kind == 2:
            K = 128 * int(rng.integers(1, 65))          # whole tiles
        else:
            K = 16 * int(rng.integers(513, 1400))       # several K chunks
        out.append((N, K, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("N,K,seed", shapes(2024, 24))
def test_random_gemv_and_gemm(N, K, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 17))
    n_big = int(rng.integers(17, 150))
    say("random", N, K, n, n_big)
    W = inputs.weights_f32(N, K, seed % 100000)
    if rng.integers(0, 3) == 0:
        W = inputs.add_zero_and_outlier_blocks(W, seed % 99991)
    codes, scales, g = O.quantize(W)
    pw = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                        g, N, K)
    X = inputs.activations_bf16(n_big, K, seed % 77777, row_scale=bool(rng.integers(0, 2)))
    Yref, Aref = O.gemv(codes, scales, g, X)
    check(y_bits(nv.gemv(pw, x_to_dev(X[:n]))), Yref[:n], Aref[:n], "gemv %dx%d n=%d" % (N, K, n))
    check(y_bits(nv.gemm(pw, x_to_dev(X))), Yref, Aref, "gemm %dx%d n=%d" % (N, K, n_big))
    # K parts: the library's choice, and a random valid part count
    T = -(-K // 128)
    valid = [k for k in range(1, min(T, 64) + 1)
             if (k - 1) * -(-T // k) < T and (k == 1 or -(-T // k) <= 64)]
    ks = int(valid[int(rng.integers(0, len(valid)))])
    for k in (0, ks):
        check(y_bits(nv.gemv_ws(pw, x_to_dev(X[:n]), k)), Yref[:n], Aref[:n],
              "gemv_ws %dx%d n=%d ks=%d" % (N, K, n, k))


@pytest.mark.parametrize("seed", list(range(8)))
def test_random_fused_qkv_splits(seed):
    rng = np.random.default_rng(500 + seed)
    rows = [int(v) for v in rng.integers(0, 300, 3)]
    if sum(rows) == 0:
        rows[0] = 1
    N = sum(rows)
    K = 16 * int(rng.integers(1, 400))
    n = int(rng.integers(1, 17))
    # projections land at permuted places in the token row, with random gaps
    order = rng.permutation(3)
    pos, off = 0, [0, 0, 0]
    for j in order:
        pos += int(rng.integers(0, 40))
        off[int(j)] = pos
        pos += rows[int(j)]
    ldy = pos + int(rng.integers(0, 40))
    say("qkv split", rows, off, ldy, K, n)
    W = inputs.weights_f32(N, K, 900 + seed)
    codes, scales, g = O.quantize(W)
    pw = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                        g, N, K)
    X = inputs.activations_bf16(n, K, 950 + seed)
    out = torch.full((n, ldy), 5.0, dtype=torch.bfloat16, device="cuda")
    Y = y_bits(nv.gemv_qkv(pw, x_to_dev(X), rows, off, ldy, out=out))
    Yref, Aref = O.gemv(codes, scales, g, X)
    mask = np.ones(ldy, dtype=bool)
    start = 0
    for p in range(3):
        check(Y[:, off[p]:off[p] + rows[p]], Yref[:, start:start + rows[p]], Aref[:, start:start + rows[p]],
              "projection %d" % p)
        mask[off[p]:off[p] + rows[p]] = False
        start += rows[p]
    assert (O.bf16_bits_to_f64(Y[:, mask]) == 5.0).all()


def big_shapes(seed, count):
    """Row counts that give every workgroup several row groups (the ring refills
    between them), with K drawn like shapes()."""
    rng = np.random.default_rng(seed)
    out = []
    for N0, K0, s in shapes(seed + 1, count):
        N = int(rng.integers(4000, 12000))
        out.append((N, K0, s))
    return out


@pytest.mark.parametrize("N,K,seed", big_shapes(4048, 16))
def test_random_multi_rowgroup(N, K, seed):
    """One-launch and K-part GEMV on N rows spread as 1-3 row groups per
    workgroup, checked on a sample of rows: every 16-row group of the first and
    last workgroup-sized stretch and a stride through the rest."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 17))
    say("random multi-rowgroup", N, K, n)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x28, 0x48, size=(N, K // 16), dtype=np.uint8)
    g = 1.0 / 128
    pw = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                        g, N, K)
    X = inputs.activations_bf16(n, K, seed % 77777, row_scale=bool(rng.integers(0, 2)))
    rows = np.array(sorted(set(list(range(0, min(N, 160))) + list(range(max(0, N - 160), N))
                           + list(range(0, N, 37)))))
    Yref, Aref = O.gemv(np.ascontiguousarray(codes[rows]), np.ascontiguousarray(scales[rows]), g, X)
    Y = y_bits(nv.gemv(pw, x_to_dev(X)))
    check(Y[:, rows], Yref, Aref, "gemv %dx%d n=%d" % (N, K, n))
    T = -(-K // 128)
    valid = [k for k in range(2, min(T, 64) + 1) if (k - 1) * -(-T // k) < T and -(-T // k) <= 64]
    if valid:
        ks = int(valid[int(rng.integers(0, len(valid)))])
        Yk = y_bits(nv.gemv_ws(pw, x_to_dev(X), ks))
        check(Yk[:, rows], Yref, Aref, "gemv_ws %dx%d n=%d ks=%d" % (N, K, n, ks))
