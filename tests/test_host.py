"""Host-side checks of the HIP library (no GPU needed): the library loads and
exports every symbol include/nvfp4.h declares, the pure host functions, and
argument validation that must fail before any HIP call."""
import ctypes

import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import nvfp4_weight_only_02_amd as nv
from nvfp4_weight_only_02_amd import metrics


def test_library_exports_every_header_symbol():
    names = nv.header_functions()
    assert len(names) >= 11
    L = nv.lib()
    for name in names:
        assert hasattr(L, name), name
    # the measurement aids live in their own library and header only
    assert not any("probe" in name or name in ("nvfp4_block_rate", "nvfp4_read_stream") for name in names)
    assert not hasattr(L, "nvfp4_probe_read_stream") and not hasattr(L, "nvfp4_read_stream")


def test_probe_library_exports_every_probe_header_symbol():
    from nvfp4_weight_only_02_amd import probes
    names = nv.header_functions(probes.HEADER_PATH)
    assert names == ["nvfp4_probe_block_rate", "nvfp4_probe_empty", "nvfp4_probe_read_stream", "nvfp4_probe_x_stage"]
    P = probes.lib()
    for name in names:
        assert hasattr(P, name), name


def test_strerror_names_every_status():
    for code, name in nv.STATUS.items():
        assert nv.strerror(code) and nv.strerror(code) != "unknown status"
    assert nv.strerror(99) == "unknown status"


def test_packed_sizes():
    assert nv.packed_codes_bytes(16384, 5120) == 16384 * 5120 // 2
    assert nv.packed_scales_bytes(16384, 5120) == 16384 * 5120 // 16
    # rows padded to 16, K to 128
    assert nv.packed_codes_bytes(17, 144) == 32 * 256 // 2
    assert nv.packed_scales_bytes(17, 144) == 32 * 256 // 16
    assert nv.packed_codes_bytes(16, 24) == 0 and nv.packed_codes_bytes(0, 16) == 0


def test_greedy_schedule_pins_from_the_pages(golden):
    case = golden["greedy_schedule"]
    for n, tiles in zip(case["n"], case["tiles"]):
        assert nv.schedule_greedy(n, 3) == tiles
    assert len(nv.schedule_greedy(8, 3)) == 3          # n=8 costs 3 weight reads
    assert len(nv.schedule_greedy(16, 3)) == 6


def test_dispatcher_schedule_reads_weights_once():
    for n in range(1, 17):
        assert nv.schedule(n, 16384, 5120) == [n]
    with pytest.raises(nv.Nvfp4Error):
        nv.schedule(17, 16, 16)
    with pytest.raises(nv.Nvfp4Error):
        nv.schedule_greedy(0, 3)


def test_launch_geometry_fills_the_chip():
    # one workgroup per compute unit per round, ranges as even as N allows:
    # every workgroup streams the same number of 16-row groups
    assert nv.launch_geometry(16, 16384, 5120) == (256, 8, 5)    # 1024 row groups: 4 each
    assert nv.launch_geometry(1, 14336, 5120) == (224, 8, 5)     # 896 row groups: 4 each
    assert nv.launch_geometry(16, 5120, 6144) == (160, 8, 6)     # 320 row groups: 2 each
    assert nv.launch_geometry(1, 1024, 1024) == (64, 8, 1)
    wg, waves, tpw = nv.launch_geometry(1, 37, 144)     # ragged: 3 row groups, 2 tiles
    assert wg == 3 and waves * tpw >= 2


@settings(max_examples=400, deadline=None)
@given(N=st.integers(1, 1 << 22), T=st.integers(1, 2048), tail=st.sampled_from([0, 16, 112]),
       n=st.integers(1, 16))
def test_launch_geometry_rule_holds_everywhere(N, T, tail, n):
    """For any shape: at most one workgroup per compute unit per round, the
    minimal number of rounds, the fewest workgroups that keep it, 8 waves, and
    a wave's K-slice of ceil(T / 8) tiles in one pass (T <= 64) or of at most
    7 tiles per chunk pass beyond."""
    K = 128 * T - tail
    if K < 16:
        return
    wg, waves, mt = nv.launch_geometry(n, N, K)
    RG = -(-N // 16)
    rounds = -(-RG // 256)
    assert waves == 8 and 1 <= wg <= 256
    assert -(-RG // wg) == rounds
    assert wg == 1 or -(-RG // (wg - 1)) > rounds
    if T <= 64:
        assert mt == -(-T // 8)
    else:
        kc = -(-T // 56)
        assert mt == -(-T // (8 * kc)) and mt <= 7


def _kparts_by_definition(N, K):
    # K parts by the stated rule: one while the 128-column tiles fit one pass
    # (64 tiles); beyond, the count (at most 64, no empty part, at most 64
    # tiles per part) minimising ceil(ks * row_groups / 256) * tiles_per_part,
    # the fewest on a tie
    T = -(-K // 128)
    RG = -(-N // 16)
    if T <= 64:
        return 1
    best = None
    for ks in range(2, min(T, 64) + 1):
        tp = -(-T // ks)
        if (ks - 1) * tp >= T or tp > 64:
            continue
        cost = -(-(ks * RG) // 256) * tp
        if best is None or cost < best[0]:
            best = (cost, ks)
    return best[1]


def test_kparts_policy():
    assert nv.gemv_kparts(5120, 17408) == 4          # dense FFN down: 4 parts of 34 tiles, 5 rounds
    for N, K in [(14336, 5120), (16384, 5120), (5120, 6144), (1024, 1024), (2048, 8192), (37, 144)]:
        assert nv.gemv_kparts(N, K) == 1             # one pass: never split
    assert nv.gemv_kparts(40, 1 << 18) == 64
    for N in (1, 16, 100, 333, 5120, 8192, 40000):
        for K in (8208, 9216, 12304, 17408, 28672, 40000, 1 << 18):
            assert nv.gemv_kparts(N, K) == _kparts_by_definition(N, K), (N, K)
    with pytest.raises(nv.Nvfp4Error):
        nv.gemv_kparts(16, 40)
    with pytest.raises(nv.Nvfp4Error):
        nv.gemv_kparts(0, 16)


def test_workspace_bytes():
    assert nv.gemv_workspace_bytes(16, 5120, 17408) == 4 * 16 * 5120 * 4
    assert nv.gemv_workspace_bytes(3, 5120, 17408, 2) == 2 * 3 * 5120 * 4
    assert nv.gemv_workspace_bytes(16, 14336, 5120) == 0      # policy: one part
    assert nv.gemv_workspace_bytes(16, 5120, 17408, 1) == 0
    assert nv.gemv_workspace_bytes(17, 5120, 17408) == 0      # invalid n
    assert nv.gemv_workspace_bytes(1, 5120, 17400) == 0       # invalid K


def test_byte_model_matches_the_pages(golden):
    b = golden["byte_model"]
    assert metrics.algorithmic_bytes(b["n"], b["N"], b["K"]) == b["bytes"]
    moved = b["us"] * 1e-6 * b["frac"] * b["GBps"] * 1e9
    assert abs(moved / b["bytes"] - 1) < 1e-3


FAKE = 0x100000   # 16-byte aligned, never dereferenced: every case below fails validation


@pytest.mark.parametrize("args,status", [
    ((0, FAKE, 1.0, FAKE, FAKE, 1, 16, 16), 1),          # null Wq
    ((FAKE, FAKE, 1.0, 0, FAKE, 1, 16, 16), 1),          # null X
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 0, 16, 16), 2),       # n = 0
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 17, 16, 16), 2),      # n > 16
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 1, 0, 16), 2),        # N = 0
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, 24), 4),       # K % 16
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, (1 << 18) + 16), 4),  # K beyond 32-bit buffer offsets
    ((FAKE + 8, FAKE, 1.0, FAKE, FAKE, 1, 16, 16), 3),   # Wq misaligned
    ((FAKE, FAKE, 1.0, FAKE + 2, FAKE, 1, 16, 16), 3),   # X misaligned
    ((FAKE, FAKE, 1.0, FAKE + 8, FAKE, 1, 16, 16), 3),   # X not 16-byte aligned
    ((FAKE, FAKE, 1.0, FAKE, FAKE + 1, 1, 16, 16), 3),   # Y misaligned
])
def test_gemv_validation(args, status):
    assert nv.lib().nvfp4_gemv(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((0, 16, 8, 0, 1 << 20), 1),                  # null sink
    ((2, 16, 8, FAKE, 1 << 20), 2),               # unknown path
    ((1, 3, 8, FAKE, 1 << 20), 2),                # n not one of 1, 2, 4, 8, 12, 16
    ((0, 16, 7, FAKE, 1 << 20), 2),               # fewer than one group of 8 blocks
    ((0, 16, 8, FAKE, 256 * 512 * 4 - 4), 2),     # sink one float short
    ((1, 8, 8, FAKE + 2, 1 << 20), 3),            # sink misaligned
])
def test_block_rate_validation(args, status):
    from nvfp4_weight_only_02_amd import probes
    assert probes.lib().nvfp4_probe_block_rate(*args, None) == status


WS = (FAKE, FAKE, 1.0, FAKE, FAKE)


@pytest.mark.parametrize("tail,status", [
    ((1, 16, 17408, 4, 0, 1 << 20), 8),                 # null workspace
    ((1, 16, 17408, 4, FAKE, 4 * 16 * 4 - 4), 8),       # workspace one float short
    ((2, 5120, 17408, 0, FAKE, 4 * 2 * 5120 * 4 - 1), 8),  # policy (4 parts) needs more
    ((1, 16, 17408, 4, FAKE + 8, 1 << 20), 3),          # workspace misaligned
    ((1, 16, 17408, -1, FAKE, 1 << 20), 2),             # ks < 0
    ((1, 16, 17408, 65, FAKE, 1 << 20), 2),             # ks beyond 64
    ((1, 16, 256, 3, FAKE, 1 << 20), 4),                # 2 tiles: a third part would be empty
    ((1, 16, 1152, 4, FAKE, 1 << 20), 4),               # 9 tiles in parts of 3: the 4th would be empty
    ((1, 16, 17408, 2, FAKE, 1 << 20), 4),              # 68 tiles per part: longer than one pass
    ((0, 16, 17408, 4, FAKE, 1 << 20), 2),              # n = 0
    ((1, 16, 17400, 4, FAKE, 1 << 20), 4),              # K % 16
])
def test_gemv_ws_validation(tail, status):
    assert nv.lib().nvfp4_gemv_ws(*WS, *tail, None) == status


@pytest.mark.parametrize("args,status", [
    ((0, FAKE, 1.0, FAKE, FAKE, 17, 16, 16), 1),                    # null Wq
    ((FAKE, FAKE, 1.0, FAKE, 0, 17, 16, 16), 1),                    # null Y
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 0, 16, 16), 2),                  # n = 0
    ((FAKE, FAKE, 1.0, FAKE, FAKE, (1 << 20) + 1, 16, 16), 2),      # n beyond NVFP4_MAX_GEMM_TOKENS
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 17, -1, 16), 2),                 # N < 1
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 17, 16, 40), 4),                 # K % 16
    ((FAKE, FAKE, 1.0, FAKE, FAKE, 17, 16, (1 << 18) + 16), 4),     # K too long
    ((FAKE, FAKE + 4, 1.0, FAKE, FAKE, 17, 16, 16), 3),             # Wscale misaligned
    ((FAKE, FAKE, 1.0, FAKE + 8, FAKE, 17, 16, 16), 3),             # X not 16-byte aligned
    ((FAKE, FAKE, 1.0, FAKE, FAKE + 1, 17, 16, 16), 3),             # Y misaligned
])
def test_gemm_validation(args, status):
    assert nv.lib().nvfp4_gemm(*args, None) == status


def test_gemm_geometry_rule():
    # token tile: smallest of 32 / 64 / 128 holding n (capped at 128)
    assert nv.gemm_geometry(17, 14336, 5120)[1] == 32
    assert nv.gemm_geometry(64, 14336, 5120)[1] == 64
    assert nv.gemm_geometry(65, 14336, 5120)[1] == 128
    assert nv.gemm_geometry(1000, 14336, 5120)[1] == 128
    # row tile: 256 rows (8 waves) once its grid gives at least half of the
    # 256 compute units a workgroup, else 64 rows (4 waves, two per unit).
    # Fused QKV, 896 row groups = 56 tiles of 256 rows:
    assert nv.gemm_geometry(100, 14336, 5120) == (64, 128, 224, 1)     # 56 workgroups: under half
    # 2 tiles of 128 tokens give 112 (under half), 4 of 64 tokens 224: 64-token tiles, 256 rows
    assert nv.gemm_geometry(256, 14336, 5120) == (256, 64, 56, 4)
    assert nv.gemm_geometry(160, 14336, 5120) == (256, 64, 56, 3)
    # one 128-token tile (56) and 2 of 64 tokens (112) are both under half: 64 rows x 128 tokens
    assert nv.gemm_geometry(128, 14336, 5120) == (64, 128, 224, 1)
    assert nv.gemm_geometry(320, 14336, 5120) == (256, 96, 56, 4)      # 96-token tiles: 224 in one round
    assert nv.gemm_geometry(512, 14336, 5120) == (256, 128, 56, 4)     # 224
    assert nv.gemm_geometry(1024, 14336, 5120) == (256, 128, 56, 8)    # 448
    # 16384 rows: 128-token tiles give 128 workgroups (half), 64-token tiles 256 in one round
    assert nv.gemm_geometry(256, 16384, 5120) == (256, 64, 64, 4)
    assert nv.gemm_geometry(640, 14336, 5120) == (256, 96, 56, 7)      # 392 in two rounds of 96 tokens
    assert nv.gemm_geometry(2048, 14336, 5120) == (256, 128, 56, 16)
    assert nv.gemm_geometry(128, 16384, 5120) == (64, 128, 256, 1)
    # 5120 rows (20 tiles of 256 rows): 7 token tiles give 140 workgroups, 6 give 120
    assert nv.gemm_geometry(896, 5120, 6144) == (256, 96, 20, 10)
    assert nv.gemm_geometry(768, 5120, 6144) == (256, 64, 20, 12)      # 6 x 128 tokens: 120; 12 x 64: 240
    assert nv.gemm_geometry(300, 5120, 6144) == (64, 128, 80, 3)       # neither reaches half
    # 16384 rows, one 128-token tile: 64 workgroups of 256 rows; 64-token tiles would reach half,
    # but with a single 128-token tile the 64-row token-split tile is kept
    assert nv.gemm_geometry(128, 16384, 5120) == (64, 128, 256, 1)
    # 34816 rows (136 tiles): the 256-row tile is wide enough at one token tile
    assert nv.gemm_geometry(40, 34816, 5120) == (256, 64, 136, 1)
    for n, N in ((17, 1), (300, 37), (5000, 100), (1 << 20, 16)):
        r, t, gx, gy = nv.gemm_geometry(n, N, 144)
        assert r in (64, 256) and gx * r >= N and gy * t >= n and (gx - 1) * r < N
    with pytest.raises(nv.Nvfp4Error):
        nv.gemm_geometry(0, 16, 16)


@pytest.mark.parametrize("args,status", [
    ((0, 0, 16, 16, FAKE, FAKE, FAKE), 1),            # null W
    ((FAKE, 0, 16, 16, FAKE, 0, FAKE), 1),            # null packed scales
    ((FAKE, 2, 16, 16, FAKE, FAKE, FAKE), 2),         # unknown dtype
    ((FAKE, 0, 0, 16, FAKE, FAKE, FAKE), 2),          # N = 0
    ((FAKE, 1, 16, 40, FAKE, FAKE, FAKE), 4),         # K % 16
    ((FAKE + 8, 0, 16, 16, FAKE, FAKE, FAKE), 3),     # W not 16-byte aligned
    ((FAKE, 0, 16, 16, FAKE + 4, FAKE, FAKE), 3),     # packed codes misaligned
    ((FAKE, 1, 16, 16, FAKE, FAKE, FAKE + 2), 3),     # tensor scale misaligned
])
def test_quantize_packed_validation(args, status):
    assert nv.lib().nvfp4_quantize_packed(*args, None) == status


def test_qkv_validation():
    L = nv.lib()
    rows = (ctypes.c_int32 * 3)(32, 16, 16)
    off = (ctypes.c_int64 * 3)(0, 32, 48)
    assert L.nvfp4_gemv_qkv(FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, None, off, 64, None) == 1
    assert L.nvfp4_gemv_qkv(FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, rows, off, 63, None) == 2   # ldy too small
    overlap = (ctypes.c_int64 * 3)(0, 16, 48)
    assert L.nvfp4_gemv_qkv(FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, rows, overlap, 64, None) == 2
    neg = (ctypes.c_int32 * 3)(32, -1, 16)
    assert L.nvfp4_gemv_qkv(FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, neg, off, 64, None) == 2
    assert L.nvfp4_gemv_qkv(FAKE, FAKE, 1.0, FAKE, FAKE, 0, 16, rows, off, 64, None) == 2


def test_sched_validation():
    L = nv.lib()
    bad = [(ctypes.c_uint8 * 2)(3, 3), 2, 5]       # widths sum to 6, n = 5
    assert L.nvfp4_gemv_sched(FAKE, FAKE, 1.0, FAKE, FAKE, 5, 16, 16, bad[0], 2, None) == 5
    zero = (ctypes.c_uint8 * 2)(5, 0)
    assert L.nvfp4_gemv_sched(FAKE, FAKE, 1.0, FAKE, FAKE, 5, 16, 16, zero, 2, None) == 5
    assert L.nvfp4_gemv_sched(FAKE, FAKE, 1.0, FAKE, FAKE, 5, 16, 16, None, 1, None) == 5
    assert L.nvfp4_gemv_sched(FAKE, FAKE, 1.0, FAKE, FAKE, 5, 16, 24, zero, 2, None) == 4


def test_quantize_and_pack_validation():
    L = nv.lib()
    assert L.nvfp4_quantize(0, 16, 16, FAKE, FAKE, FAKE, None) == 1
    assert L.nvfp4_quantize(FAKE, 16, 24, FAKE, FAKE, FAKE, None) == 4
    assert L.nvfp4_quantize(FAKE + 4, 16, 16, FAKE, FAKE, FAKE, None) == 3
    assert L.nvfp4_quantize(FAKE, 0, 16, FAKE, FAKE, FAKE, None) == 2
    assert L.nvfp4_pack(FAKE, FAKE, 16, 16, FAKE + 8, FAKE, None) == 3
    assert L.nvfp4_pack(FAKE, 0, 16, 16, FAKE, FAKE, None) == 1
    assert L.nvfp4_pack(FAKE, FAKE, 16, 20, FAKE, FAKE, None) == 4


def test_gemv_ws_static_validation():
    """The no-allocation K-part entry point refuses, before any HIP call,
    what does not fit its fixed 8 MiB scratch, and validates as gemv_ws."""
    L = nv.lib()
    assert nv.gemv_static_scratch_bytes() == 8 << 20
    # 16 tokens x 65536 rows x 4 parts x 4 bytes = 16 MiB > 8 MiB
    assert L.nvfp4_gemv_ws_static(FAKE, FAKE, 1.0, FAKE, FAKE, 16, 65536, 17408, 4, None) == 9
    assert L.nvfp4_gemv_ws_static(FAKE, FAKE, 1.0, FAKE, FAKE, 16, 32768, 17408, 5, None) == 9
    assert L.nvfp4_gemv_ws_static(0, FAKE, 1.0, FAKE, FAKE, 1, 16, 17408, 4, None) == 1
    assert L.nvfp4_gemv_ws_static(FAKE, FAKE, 1.0, FAKE, FAKE, 17, 16, 17408, 4, None) == 2
    assert L.nvfp4_gemv_ws_static(FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, 17408, 65, None) == 2
    assert L.nvfp4_gemv_ws_static(FAKE, FAKE, 1.0, FAKE, FAKE, 1, 16, 17408, 2, None) == 4
    assert nv.strerror(9) != "unknown status"


def test_probe_validation():
    from nvfp4_weight_only_02_amd import probes
    P = probes.lib()
    assert P.nvfp4_probe_read_stream(None, 1024, FAKE, None) == 1
    assert P.nvfp4_probe_read_stream(FAKE, 1024, None, None) == 1
    assert P.nvfp4_probe_read_stream(FAKE, 0, FAKE, None) == 2
    assert P.nvfp4_probe_read_stream(FAKE, 1000, FAKE, None) == 2
    assert P.nvfp4_probe_read_stream(FAKE + 8, 1024, FAKE, None) == 3
    assert P.nvfp4_probe_empty(0, None) == 2
    assert P.nvfp4_probe_empty(65537, None) == 2
    # nvfp4_probe_x_stage(X, n, K, workgroups, reps, mode, sink, stream)
    assert P.nvfp4_probe_x_stage(None, 16, 5120, 256, 4, 0, FAKE, None) == 1
    assert P.nvfp4_probe_x_stage(FAKE, 16, 5120, 256, 4, 0, None, None) == 1
    for bad in [(0, 5120, 256, 4, 0), (17, 5120, 256, 4, 0), (16, 5000, 256, 4, 0), (16, 8320, 256, 4, 0),
                (16, 0, 256, 4, 0), (16, 5120, 0, 4, 0), (16, 5120, 65537, 4, 0), (16, 5120, 256, 0, 0),
                (16, 5120, 256, 1025, 0), (16, 5120, 256, 4, 2)]:
        assert P.nvfp4_probe_x_stage(FAKE, *bad, FAKE, None) == 2, bad
    assert P.nvfp4_probe_x_stage(FAKE + 8, 16, 5120, 256, 4, 0, FAKE, None) == 3


def test_row_counts_near_int_max_do_not_overflow():
    """Row groups are rounded up in 64-bit arithmetic: N = INT_MAX has
    2^27 sixteen-row groups, and the host functions stay defined there."""
    big = 2**31 - 1
    assert nv.packed_codes_bytes(big, 128) == 2**27 * 16 * 64
    assert nv.packed_scales_bytes(big, 128) == 2**27 * 16 * 8
    wg, waves, tpw = nv.launch_geometry(1, big, 128)
    assert wg == 256 and waves == 8 and tpw == 1
    assert nv.gemv_variant(1, big, 128) == (1, 1, 0, 1, 1)
    assert nv.gemv_kparts(big, 17408) >= 1


def test_gemv_sched_checks_the_output_shape_before_the_library(monkeypatch):
    """An output of the wrong shape is refused on the host, before the C call
    (which could not know the buffer's size)."""
    import torch

    def no_lib():
        raise AssertionError("the library must not be called")
    monkeypatch.setattr(nv, "_dev", lambda t, dtype, name: t)
    monkeypatch.setattr(nv, "lib", no_lib)
    w = nv.PackedWeight(torch.zeros(512, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8), 1.0, 16, 64)
    X = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must be"):
        nv.gemv_sched(w, X, [3, 1], out=torch.zeros((3, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        nv.gemv(w, X, out=torch.zeros((4, 17), dtype=torch.bfloat16))


def test_build_refuses_spilling_gemv_kernels():
    """The build check that keeps the GEMV kernels free of spills (their loads
    are inline assembly waited for by hand; a spill could copy a register
    whose load is still in flight)."""
    from nvfp4_weight_only_02_amd import build
    ok = ("x.hip:1:1: remark: Function Name: _ZN12nvfp4_gemv_kernelILi5E [-Rpass]\n"
          "x.hip:1:1: remark:     VGPRs: 170 [-Rpass]\n"
          "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass]\n"
          "x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass]\n"
          "x.hip:1:1: remark: Function Name: _ZN12other_kernel [-Rpass]\n"
          "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 64 [-Rpass]\n")
    build.check_resources(ok)
    bad = ok + ("x.hip:1:1: remark: Function Name: _ZN12nvfp4_gemv_kernelILi6E [-Rpass]\n"
                "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 68 [-Rpass]\n"
                "x.hip:1:1: remark:     VGPRs Spill: 16 [-Rpass]\n")
    with pytest.raises(RuntimeError, match="must not spill"):
        build.check_resources(bad)


def test_device_rule_of_the_binding():
    """Every tensor of a call and its stream must be on the current device,
    where the library launches; anything else is refused before the call."""
    import torch
    d0, d1 = torch.device("cuda", 0), torch.device("cuda", 1)
    nv.check_devices([d0, d0, d0], 0, d0)
    nv.check_devices([], 0, d0)
    for devices, current, stream_device in [([d0, d1], 0, d0), ([d1, d1], 0, d1), ([d0], 0, d1),
                                            ([torch.device("cpu")], 0, d0), ([d1], 1, d0)]:
        with pytest.raises(ValueError):
            nv.check_devices(devices, current, stream_device)


@settings(max_examples=300, deadline=None)
@given(N=st.integers(-3, 2**31 - 1), K=st.integers(-40, 300000), n=st.integers(-2, 40), ks=st.integers(-2, 80))
def test_host_queries_are_total_and_consistent(N, K, n, ks):
    """The pure host functions (no device, no launch) answer every argument
    set, including sizes near INT_MAX, without overflow: packed sizes follow
    the tile layout, the part count is 1..64 for every valid shape, the
    workspace is parts * n * N * 4 bytes, a schedule covers exactly n tokens,
    and geometry is reported only for shapes nvfp4_gemv accepts."""
    L = nv.lib()
    shape_ok = N >= 1 and 16 <= K <= 262144 and K % 16 == 0
    cb, sb = L.nvfp4_packed_codes_bytes(N, K), L.nvfp4_packed_scales_bytes(N, K)
    if N >= 1 and K >= 1 and K % 16 == 0:
        rg, t = -(-N // 16), -(-K // 128)
        assert (cb, sb) == (rg * t * 1024, rg * t * 128)
    else:
        assert (cb, sb) == (0, 0)
    kp = L.nvfp4_gemv_kparts(N, K)
    if shape_ok:
        assert 1 <= kp <= 64
    else:
        assert kp < 0
    wb = L.nvfp4_gemv_workspace_bytes(n, N, K, ks)
    parts = kp if ks == 0 else ks
    if shape_ok and 1 <= n <= 16 and parts > 1 and wb:
        assert wb == parts * n * N * 4
    if not shape_ok or not 1 <= n <= 16:
        assert wb == 0
    buf = (ctypes.c_uint8 * 16)()
    cnt = L.nvfp4_schedule(n, N, K, buf, 16)
    if 1 <= n <= 16 and shape_ok:
        assert cnt >= 1 and sum(buf[:cnt]) == n and all(1 <= w <= 16 for w in buf[:cnt])
    else:
        assert cnt < 0
    wg, wv, tpw = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    status = L.nvfp4_launch_geometry(n, N, K, ctypes.byref(wg), ctypes.byref(wv), ctypes.byref(tpw))
    if status == 0:
        assert shape_ok and 1 <= n <= 16
        assert 1 <= wg.value <= 256 and wv.value == 8 and 1 <= tpw.value <= 8
    elif shape_ok and 1 <= n <= 16:
        assert status == 4   # SHAPE: a workgroup's codes beyond a 32-bit buffer offset



def test_committed_counters_match_the_built_kernel_code():
    """The HBM counter summaries the bench reads were taken on exactly the
    GEMV machine code built here (else the bench would report no traffic)."""
    import json
    import os
    import bench
    code = bench.kernel_code_hash()
    assert code is not None
    folder = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    names = [f for f in os.listdir(folder) if f.endswith("_counters.json")]
    assert names
    for name in names:
        with open(os.path.join(folder, name)) as f:
            assert json.load(f)["kernel_code_sha256_16"] == code, name


_PTRS = st.sampled_from([None, FAKE, FAKE + 2, FAKE + 8])
_INTS = st.one_of(st.integers(-5, 70), st.integers(-(2**31), 2**31 - 1), st.sampled_from([16, 128, 5120, 262144, 262160]))


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="arguments can pass validation: only safe where no GPU would run the launch")
@settings(max_examples=300, deadline=None)
@given(ptrs=st.lists(_PTRS, min_size=6, max_size=6), ints=st.lists(_INTS, min_size=8, max_size=8),
       size=st.integers(0, 2**40))
def test_launching_entry_points_never_crash_on_host(ptrs, ints, size):
    """Every entry point that launches work answers any argument set with a
    status: a validation error, or (here, with no GPU) NVFP4_ERR_DEVICE.  It
    never returns OK without a device and never crashes on the host."""
    L = nv.lib()
    a, b, x, y, ws, sink = ptrs
    n, N, K, ks, r0, r1, r2, ldy = ints
    statuses = set(range(1, 10))
    rows = (ctypes.c_int32 * 3)(*(max(-(2**31), min(2**31 - 1, v)) for v in (r0, r1, r2)))
    offs = (ctypes.c_int64 * 3)(r2, r0, r1)
    widths = (ctypes.c_uint8 * 4)(*(v & 0xFF for v in (n, ks, r0, r1)))
    calls = [
        L.nvfp4_gemv(a, b, 1.0, x, y, n, N, K, None),
        L.nvfp4_gemv_ws(a, b, 1.0, x, y, n, N, K, ks, ws, size, None),
        L.nvfp4_gemv_ws_static(a, b, 1.0, x, y, n, N, K, ks, None),
        L.nvfp4_gemv_qkv(a, b, 1.0, x, y, n, K, rows, offs, ldy, None),
        L.nvfp4_gemv_sched(a, b, 1.0, x, y, n, N, K, widths, ks & 3, None),
        L.nvfp4_gemm(a, b, 1.0, x, y, n, N, K, None),
        L.nvfp4_pack(a, b, N, K, x, y, None),
        L.nvfp4_quantize(a, N, K, x, y, sink, None),
        L.nvfp4_quantize_packed(a, ks & 1, N, K, x, y, sink, None),
    ]
    for i, status in enumerate(calls):
        assert status in statuses, (i, status)
