"""A broad seeded sweep of the GPU path against the oracle.

Each case draws a shape (N up to 12000 rows, K up to 35200 columns), a token
count, a tensor scale, scale bytes over the E4M3 range and one of the two
activation recipes, then runs every entry point on the same weight:
  * nvfp4_gemv (n tokens),
  * nvfp4_gemv_ws with a random valid part count,
  * nvfp4_gemv_qkv with a random three-way row split written at rotated
    offsets,
  * nvfp4_gemm with a wider token count (17 .. 299),
and checks sampled rows (the first and last 48 and 64 random ones) against
the oracle's fp64 sums with the GEMV tolerance.
"""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from nvfp4_weight_only_02_amd import inputs

pytestmark = pytest.mark.gpu

CASES = 120


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    nv.lib()
    yield
    torch.cuda.synchronize()


def x_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def y_bits(Y: torch.Tensor) -> np.ndarray:
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def within(Yb, Yref, Aref):
    y = O.bf16_bits_to_f64(Yb)
    tol = O.tolerance(Yref, Aref)
    err = np.abs(y - Yref)
    return bool((err <= tol).all()), float(np.max(err / tol))


def valid_part_counts(K: int) -> list:
    T = -(-K // 128)
    return [ks for ks in range(1, min(T, 64) + 1)
            if (ks - 1) * -(-T // ks) < T and (ks == 1 or -(-T // ks) <= 64)]


def draw(rng):
    N = int(rng.choice([rng.integers(1, 64), rng.integers(64, 2000), rng.integers(2000, 12000)]))
    K = 16 * int(rng.choice([rng.integers(1, 64), rng.integers(64, 520), rng.integers(520, 2200)]))
    return N, K


def test_seeded_sweep_of_every_entry_point():
    rng = np.random.default_rng(20261202)
    failures = []
    for case in range(CASES):
        N, K = draw(rng)
        n = int(rng.integers(1, 17))
        codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        scales = rng.integers(0x20, 0x50, size=(N, K // 16), dtype=np.uint8)
        g = float(2.0 ** -int(rng.integers(4, 10)))
        w = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                           g, N, K)
        wide = int(rng.integers(17, 300))
        X = inputs.activations_bf16(wide, K, int(rng.integers(0, 1 << 30)), row_scale=bool(rng.integers(0, 2)))
        rows = np.unique(np.concatenate([np.arange(min(N, 48)), np.arange(max(0, N - 48), N),
                                         rng.integers(0, N, 64)]))
        Yref, Aref = O.gemv(codes[rows], scales[rows], g, X)
        Xd = x_dev(X)
        Xn = Xd[:n].contiguous()
        ks = int(rng.choice(valid_part_counts(K)))
        outs = {"gemv": (y_bits(nv.gemv(w, Xn)), n),
                "gemv_ws ks=%d" % ks: (y_bits(nv.gemv_ws(w, Xn, ks)), n),
                "gemm n=%d" % wide: (y_bits(nv.gemm(w, Xd)), wide)}
        if N >= 3:
            a = int(rng.integers(1, N - 1))
            b = int(rng.integers(1, N - a))
            c = N - a - b
            outs["qkv %d/%d/%d" % (a, b, c)] = (y_bits(nv.gemv_qkv(w, Xn, (a, b, c), (c, c + a, 0), N)), n)
        for name, (Yb, m) in outs.items():
            if name.startswith("qkv"):
                a_, b_, c_ = (int(v) for v in name.split()[1].split("/"))
                # undo the rotation: q at c, k at c + a, v at 0
                Yb = np.concatenate([Yb[:, c_:c_ + a_], Yb[:, c_ + a_:c_ + a_ + b_], Yb[:, :c_]], axis=1)
            ok, worst = within(Yb[:, rows], Yref[:m], Aref[:m])
            if not ok:
                failures.append("case %d %dx%d n=%d %s: worst err/tol %.3g" % (case, N, K, m, name, worst))
        del w
    assert not failures, "\n".join(failures)
