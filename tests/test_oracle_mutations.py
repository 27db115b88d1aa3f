"""Planted mistakes in a private copy of the oracle must each fail a pin.

Each mutation edits the C source of the oracle (never the product), builds it
into a temporary library and reruns the pins of test_oracle.py against it.  A
mutation that no pin catches would mean the pins leave that part of the oracle
unchecked.
"""
import ctypes
import importlib.util
import os
import subprocess

import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))

MUTATIONS = [
    ("nibble_order_swapped", "return (k % 2 == 0) ? (byte & 15) : (byte >> 4);",
     "return (k % 2 == 0) ? (byte >> 4) : (byte & 15);", 1),
    ("scale_index_per_8", "E4M3_TABLE[scales[(size_t)r * (K / 16) + k / 16]]",
     "E4M3_TABLE[scales[(size_t)r * (K / 16) + (k / 8) % (K / 16)]]", 0),
    ("gscale_dropped", "*\n                           (double)gscale;", ";", 0),
    ("e2m1_sign_lost", "-0.0, -0.5, -1.0", "-0.0, 0.5, -1.0", 1),
    ("e4m3_bias_off_by_one", "expo - 7", "expo - 6", 1),
    ("x_transposed", "X[(size_t)t * K + k]", "X[(size_t)k * n + t]", 1),
    ("abs_dropped_in_bound", "mag += fabs(p);", "mag += p;", 0),
    ("last_term_dropped", "for (int k = 0; k < K; ++k) {\n                double w",
     "for (int k = 0; k < K - 1; ++k) {\n                double w", 1),
    ("e2m1_tie_to_odd", "(err == best_err && (i % 2) == 0)", "(err == best_err && (i % 2) == 1)", 1),
    ("e4m3_tie_to_odd", "(err == best_err && (b % 2) == 0)", "(err == best_err && (b % 2) == 1)", 1),
    ("block_amax_over_15", "for (int i = 0; i < 16; ++i)\n                if (fabs",
     "for (int i = 0; i < 15; ++i)\n                if (fabs", 1),
    ("tensor_scale_448_only", "(6.0 * 448.0)", "(448.0)", 1),
]


def _load_pins():
    spec = importlib.util.spec_from_file_location("oracle_pins", os.path.join(HERE, "test_oracle.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new,count", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, count, tmp_path, golden, monkeypatch):
    src = open(O._SRC).read()
    assert old in src, "mutation anchor missing: " + name
    mutated = src.replace(old, new, count) if count else src.replace(old, new)
    c_path = tmp_path / "mut.c"
    so_path = tmp_path / "libmut.so"
    c_path.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           str(c_path), "-o", str(so_path), "-lm"])
    monkeypatch.setattr(O, "_lib", O.configure(ctypes.CDLL(str(so_path))))
    T = _load_pins()
    pins = [
        lambda: T.test_e2m1_table_closed_values(),
        lambda: T.test_e4m3_table_matches_torch_float8(),
        lambda: T.test_e2m1_rne_hand(golden),
        lambda: T.test_e4m3_rne_hand(golden),
        lambda: T.test_quantize_ties_block(golden),
        lambda: T.test_quantize_matches_exact_rational(),
        lambda: T.test_gemv_hand_blocks(golden),
        lambda: T.test_gemv_matches_numpy_matmul(33, 160, 16),
        lambda: T.test_gemv_matches_numpy_matmul(5, 48, 3),
    ]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, "no pin caught the planted mistake " + name
