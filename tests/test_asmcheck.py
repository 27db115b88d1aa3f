"""The static in-flight-register check (nvfp4_weight_only_02_amd/asmcheck.py),
no GPU: it must flag every planted read or write of a pending load's
destination in small hand-written instruction streams and in a real kernel of
the built library, stay quiet where an s_waitcnt covers the load, and find the
built library's GEMV and GEMM kernels clean."""
import os

import pytest

from nvfp4_weight_only_02_amd import asmcheck, build


def prog(text):
    """Instruction list from 'mnemonic operands' lines, 4 bytes each from 0."""
    out = []
    for i, line in enumerate(l.strip() for l in text.strip().splitlines()):
        mnem, _, ops = line.partition(" ")
        out.append((4 * i, mnem, ops.strip()))
    return out


def flagged(text):
    return [v[0] // 4 for v in asmcheck.check_function(prog(text))]


def test_read_before_wait_is_flagged():
    assert flagged("""
        buffer_load_dwordx4 v[0:3], v8, s[4:7], 0 offen
        v_add_f32_e32 v4, v1, v5
        s_endpgm""") == [1]


def test_write_before_wait_is_flagged():
    assert flagged("""
        buffer_load_dwordx4 v[0:3], v8, s[4:7], 0 offen
        v_mov_b32_e32 v2, 0
        s_endpgm""") == [1]


def test_covered_by_waitcnt():
    assert flagged("""
        buffer_load_dwordx4 v[0:3], v8, s[4:7], 0 offen
        buffer_load_dwordx4 v[4:7], v8, s[4:7], 0 offen offset:16
        s_waitcnt vmcnt(1)
        v_add_f32_e32 v9, v0, v3
        v_add_f32_e32 v10, v4, v9
        s_waitcnt vmcnt(0) lgkmcnt(0)
        v_add_f32_e32 v11, v4, v7
        s_endpgm""") == [4]


def test_stores_count_and_lds_loads_have_no_destination():
    # the store is newer than the load: vmcnt(1) retires the load
    assert flagged("""
        global_load_dwordx2 v[0:1], v[8:9], off
        global_store_short v[10:11], v12, off
        s_waitcnt vmcnt(1)
        v_add_f32_e32 v4, v0, v1
        s_endpgm""") == []
    # here the store is older: vmcnt(1) leaves the load in flight
    assert flagged("""
        global_store_short v[10:11], v12, off
        global_load_dwordx2 v[0:1], v[8:9], off
        s_waitcnt vmcnt(1)
        v_add_f32_e32 v4, v0, v1
        s_endpgm""") == [3]
    assert flagged("""
        buffer_load_dword v1, s[4:7], 0 offen lds
        v_add_f32_e32 v4, v1, v1
        s_endpgm""") == []


def test_raw_waitcnt_encoding():
    # 0x3F70: vmcnt = 0 (bits 3:0 and 15:14 clear)
    assert flagged("""
        buffer_load_dword v0, v8, s[4:7], 0 offen
        s_waitcnt 0x3f70
        v_add_f32_e32 v4, v0, v0
        s_endpgm""") == []


def test_paths_merge_conservatively():
    # the branch skips the wait: the use after the join may see the load in flight
    assert flagged("""
        buffer_load_dwordx4 v[0:3], v8, s[4:7], 0 offen
        s_cbranch_scc1 1
        s_waitcnt vmcnt(0)
        v_add_f32_e32 v4, v0, v1
        s_endpgm""") == [3]
    # a backward branch in 16-bit two's complement, as the disassembler prints
    # it: the loop's second trip reads v0 while the load of the first is in
    # flight, and loads into v0 again before that load has landed
    assert flagged("""
        v_mov_b32_e32 v9, 0
        v_add_f32_e32 v4, v0, v9
        buffer_load_dword v0, v8, s[4:7], 0 offen
        s_cbranch_scc1 65533
        s_waitcnt vmcnt(0)
        s_endpgm""") == [1, 2]
    assert flagged("""
        s_waitcnt vmcnt(0)
        v_add_f32_e32 v4, v0, v4
        buffer_load_dword v0, v8, s[4:7], 0 offen
        s_cbranch_scc1 65532
        s_waitcnt vmcnt(0)
        s_endpgm""") == []


def test_agprs_are_registers_too():
    assert flagged("""
        buffer_load_dwordx2 a[0:1], v8, s[4:7], 0 offen
        v_accvgpr_read_b32 v4, a1
        s_endpgm""") == [1]


@pytest.fixture(scope="module")
def built():
    lib = build.LIB
    if not os.path.exists(lib):
        pytest.skip("library not built")
    return asmcheck.parse(asmcheck.disassemble(lib))


def test_built_kernels_are_clean(built):
    names = [f for f in built if "nvfp4_gemv_kernel" in f or "nvfp4_gemm_kernel" in f]
    assert len([f for f in names if "gemv_kernel" in f]) >= 152
    deep = 0
    for f in names:
        st = {}
        assert asmcheck.check_function(built[f], st) == [], f
        deep = max(deep, st["max_outstanding"])
    # the analysis sees the hand-issued loads: X plus the weight ring in flight
    assert deep >= 20


def test_planted_read_in_a_real_kernel_is_flagged(built):
    name = next(f for f in built if "nvfp4_gemv_kernelILi5ELi4ELb1ELb0ELb0E" in f)
    code = built[name]
    i = next(k for k, (_, m, o) in enumerate(code) if m == "buffer_load_dwordx4")
    dest = code[i][2].split(",")[0].strip()          # e.g. v[6:9]
    first = "v" + dest[2:].split(":")[0] if dest.startswith("v[") else dest
    addr = code[i][0]
    planted = code[:i + 1] + [(addr + 2, "v_mov_b32_e32", "v200, " + first)] + code[i + 1:]
    out = asmcheck.check_function(planted)
    assert [v[0] for v in out] == [addr + 2]
