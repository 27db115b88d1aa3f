"""The GEMV kernel instantiations the dispatcher can launch, restated from its
rule, and one small call per instantiation for the GPU tests.

Each ``nvfp4_gemv_kernel<MT, NV, EXACT, CHUNKED, SPLIT>`` is compiled on its
own with its own compile-time wait counts, so every one the dispatcher can
pick gets a parity case.  The rule (what nvfp4_gemv_variant reports):
  * T = ceil(K / 128) tiles; ks K parts of tp = ceil(T / ks) tiles, none empty
    ((ks - 1) * tp < T), each at most one pass (tp <= 64) when ks > 1;
  * one pass holds 64 tiles (8 waves x 8); beyond, passes of at most 56
    (8 x 7): kc = ceil(tp / per_pass) passes, MT = ceil(tp / (8 kc)) tiles per
    wave;
  * EXACT when K is a multiple of 128 and every wave owns exactly MT tiles of
    every pass of every part (T = ks * tp, tp = kc * 8 * MT);
  * NV = ceil(n / 4); CHUNKED = kc > 1; SPLIT = ks > 1.
"""
from __future__ import annotations

MAX_K = 1 << 18
MAX_PARTS = 64


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def variant(n: int, K: int, ks: int):
    """(MT, NV, exact, passes, parts) for an explicit part count, or None when
    nvfp4_gemv_ws would refuse the shape."""
    T = cdiv(K, 128)
    if ks < 1 or ks > T or ks > MAX_PARTS:
        return None
    tp = cdiv(T, ks)
    if (ks - 1) * tp >= T or (ks > 1 and tp > 64):
        return None
    kc = cdiv(tp, 64 if tp <= 64 else 56)
    mt = cdiv(tp, 8 * kc)
    exact = K % 128 == 0 and T == ks * tp and tp == kc * 8 * mt
    return (mt, cdiv(n, 4), int(exact), kc, ks)


def kernel_of(v) -> tuple:
    """The template arguments (MT, NV, EXACT, CHUNKED, SPLIT) of a variant."""
    mt, nv, exact, kc, ks = v
    return (mt, nv, bool(exact), kc > 1, ks > 1)


def k_values(T: int):
    """K values with T tiles: a multiple of 128 and ragged tails."""
    return [K for K in (128 * T, 128 * T - 16, 128 * T - 112) if 16 <= K <= MAX_K and cdiv(K, 128) == T]


def reachable_kernels() -> set:
    """Every (MT, NV, EXACT, CHUNKED, SPLIT) some valid (n, K, ks) reaches."""
    out = set()
    for T in range(1, MAX_K // 128 + 1):
        for K in k_values(T):
            for ks in range(1, min(T, MAX_PARTS) + 1):
                v = variant(1, K, ks)
                if v is None:
                    continue
                for nv in (1, 2, 3, 4):
                    out.add(kernel_of((v[0], nv) + v[2:]))
    return out


# Rows of every coverage case: 513 row groups (the last one 8 rows), so that
# on 256 compute units each workgroup streams several row groups (the ring
# refills between them) and the last row group is ragged.
COVER_N = 8200


def coverage_cases() -> list:
    """One (N, K, n, ks) per reachable kernel, the smallest K that reaches it
    (ks = 1 where the kernel is not a K-part one); n cycles through the token
    counts of its NV so that not every case is a whole number of quads."""
    want = sorted(reachable_kernels())
    found = {}
    for T in range(1, MAX_K // 128 + 1):
        for K in k_values(T):
            for ks in range(1, min(T, MAX_PARTS) + 1):
                v = variant(1, K, ks)
                if v is None:
                    continue
                for nv in (1, 2, 3, 4):
                    key = kernel_of((v[0], nv) + v[2:])
                    if key not in found:
                        found[key] = (K, ks)
        if len(found) == len(want):
            break
    cases = []
    for j, key in enumerate(want):
        K, ks = found[key]
        nv = key[1]
        n = 4 * nv - (j % 4)
        cases.append((COVER_N, K, n, ks))
    return cases
