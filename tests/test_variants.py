"""The GEMV kernel instantiations the dispatcher can reach (no GPU): the
library's own answer (nvfp4_gemv_variant) agrees with the restated rule for
every K up to 262144 and every part count, and the GPU coverage cases reach
every instantiation once."""
import ctypes

import nvfp4_weight_only_02_amd as nv
from kernel_variants import (COVER_N, MAX_K, MAX_PARTS, cdiv, coverage_cases, k_values, kernel_of,
                             reachable_kernels, variant)


def test_dispatcher_matches_the_stated_rule_everywhere():
    L = nv.lib()
    v = (ctypes.c_int * 5)()
    checked = 0
    for T in range(1, MAX_K // 128 + 1):
        for K in k_values(T):
            for ks in range(1, MAX_PARTS + 1):
                want = variant(1, K, ks)
                st = L.nvfp4_gemv_variant(1, 64, K, ks, v)
                if want is None:
                    assert st == 4, (K, ks, st)            # NVFP4_ERR_SHAPE, as nvfp4_gemv_ws
                else:
                    assert st == 0 and tuple(v) == want, (K, ks, tuple(v), want)
                    checked += 1
    assert checked > 50000


def test_token_groups_and_default_parts():
    for n in range(1, 17):
        assert nv.gemv_variant(n, 16384, 5120)[1] == cdiv(n, 4)
    # ks = 0 is the library's part count for the shape
    for N, K in ((5120, 17408), (5120, 6144), (300, 262144), (34816, 5120)):
        ks = nv.gemv_kparts(N, K)
        assert nv.gemv_variant(16, N, K, 0) == variant(16, K, ks)
    # the decode shapes: one pass, exact, five or six tiles per wave
    assert nv.gemv_variant(16, 16384, 5120) == (5, 4, 1, 1, 1)
    assert nv.gemv_variant(16, 14336, 5120) == (5, 4, 1, 1, 1)
    assert nv.gemv_variant(1, 5120, 6144) == (6, 1, 1, 1, 1)
    assert nv.gemv_variant(8, 5120, 17408) == (6, 2, 0, 3, 1)   # 136 tiles: 3 passes of 6 per wave


def test_reachable_kernels():
    r = reachable_kernels()
    # one-pass kernels: MT 1..8, exact or not, 4 token groups; chunked: MT
    # 5..7; K parts: every one-pass MT
    assert {k[:3] for k in r if not k[3] and not k[4]} == {(mt, nv_, e) for mt in range(1, 9)
                                                          for nv_ in range(1, 5) for e in (False, True)}
    assert {k[0] for k in r if k[3]} == {5, 6, 7}
    assert not any(k[3] and k[4] for k in r)
    assert len(r) == 64 + 24 + 64


def test_coverage_cases_reach_every_kernel_once():
    cases = coverage_cases()
    got = [kernel_of(nv.gemv_variant(n, N, K, ks)) for N, K, n, ks in cases]
    assert sorted(got) == sorted(reachable_kernels())
    assert len(set(got)) == len(got)
    for N, K, n, ks in cases:
        assert N == COVER_N and 1 <= n <= 16 and K <= 16384
        # several row groups per workgroup on 256 compute units, so the
        # weight ring refills between row groups in every case
        wg, _, _ = nv.launch_geometry(n, N, K)
        assert cdiv(N, 16) > wg


def test_variant_validation():
    L = nv.lib()
    v = (ctypes.c_int * 5)()
    assert L.nvfp4_gemv_variant(1, 16, 16, 1, None) == 1
    assert L.nvfp4_gemv_variant(0, 16, 16, 1, v) == 2
    assert L.nvfp4_gemv_variant(17, 16, 16, 1, v) == 2
    assert L.nvfp4_gemv_variant(1, 0, 16, 1, v) == 2
    assert L.nvfp4_gemv_variant(1, 16, 16, -1, v) == 2
    assert L.nvfp4_gemv_variant(1, 16, 16, 65, v) == 2
    assert L.nvfp4_gemv_variant(1, 16, 24, 1, v) == 4
    assert L.nvfp4_gemv_variant(1, 16, MAX_K + 16, 1, v) == 4
    assert L.nvfp4_gemv_variant(1, 16, 128, 2, v) == 4      # more parts than tiles
