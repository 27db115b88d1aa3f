"""CPU oracle for the NVFP4 weight-only projection GEMV of batched decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(``nvfp4_weight_only_02_amd`` and its HIP library) never imports it, and it
imports nothing from the product.

Every arithmetic step lives in ``nvfp4_oracle.c`` (plain C, fp64, OpenMP over
rows); this module only marshals numpy arrays through ctypes, plus the two
purely structural helpers below (the fused-QKV scatter and the acceptance
bound).  What each function follows:

* the GEMV ``y[t][r] = sum_k x[t][k] * dequant(W)[r][k]`` -- Atlas PR #266,
  PR description ("What it does"): each token tile reads the projection weight
  once; tiling changes only the accumulation order (A/B comment, "Numeric
  identity" caveat), so the oracle evaluates the definition directly;
* the fused-QKV scatter -- same PR description, ``multi_seq/qkv.rs`` bullet: q,
  k and v rows of one fused weight land at fixed offsets of a per-sequence
  buffer (``q_proj_bytes`` / ``kv_bytes`` / ``per_seq_qkv``);
* NVFP4 bit formats -- the pages only name NVFP4; the OCP FP4 E2M1 and OCP FP8
  E4M3FN encodings are used, and the quantiser follows the stated input recipe
  (tensor scale amax/(6*448), E4M3 block scale per 16 elements, RNE).

Parity pins: ``tests/test_oracle.py``.  No function here is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def configure(L):
    """Declare the C signatures on a loaded copy of the oracle library."""
    L.oracle_e2m1.restype = ctypes.c_double
    L.oracle_e2m1.argtypes = [ctypes.c_int]
    L.oracle_e4m3.restype = ctypes.c_double
    L.oracle_e4m3.argtypes = [ctypes.c_int]
    L.oracle_bf16_rne.restype = ctypes.c_uint16
    L.oracle_bf16_rne.argtypes = [ctypes.c_double]
    L.oracle_bf16_rne_array.restype = None
    L.oracle_bf16_rne_array.argtypes = [_f64p, ctypes.c_size_t, _u16p]
    L.oracle_e2m1_rne_index.restype = ctypes.c_int
    L.oracle_e2m1_rne_index.argtypes = [ctypes.c_double]
    L.oracle_e4m3_rne.restype = ctypes.c_int
    L.oracle_e4m3_rne.argtypes = [ctypes.c_double]
    L.oracle_tensor_scale.restype = ctypes.c_float
    L.oracle_tensor_scale.argtypes = [_f32p, ctypes.c_size_t]
    L.oracle_quantize.restype = None
    L.oracle_quantize.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, _u8p, _u8p, _f32p]
    L.oracle_dequant.restype = None
    L.oracle_dequant.argtypes = [_u8p, _u8p, ctypes.c_float, ctypes.c_int, ctypes.c_int, _f64p]
    L.oracle_gemv.restype = None
    L.oracle_gemv.argtypes = [_u8p, _u8p, ctypes.c_float, _u16p, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int, _f64p, _f64p, ctypes.c_int]
    L.oracle_gemv_one.restype = ctypes.c_double
    L.oracle_gemv_one.argtypes = [_u8p, _u8p, ctypes.c_float, _u16p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, _f64p]
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_num_threads.argtypes = []
    return L


def lib():
    global _lib
    if _lib is None:
        _lib = configure(ctypes.CDLL(build()))
    return _lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---- scalar decode / encode ------------------------------------------------

def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e4m3(byte: int) -> float:
    return lib().oracle_e4m3(int(byte))


def e2m1_rne_index(q: float) -> int:
    return lib().oracle_e2m1_rne_index(float(q))


def e4m3_rne(v: float) -> int:
    return lib().oracle_e4m3_rne(float(v))


def bf16_rne(v) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_ptr(a, ctypes.c_double), a.size, _ptr(out, ctypes.c_uint16))
    return out.reshape(np.shape(v))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bit placement only, no rounding)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---- quantiser -------------------------------------------------------------

def tensor_scale(W: np.ndarray) -> float:
    a = np.ascontiguousarray(W, dtype=np.float32)
    return float(lib().oracle_tensor_scale(_ptr(a, ctypes.c_float), a.size))


def quantize(W: np.ndarray):
    """fp32 [N][K] -> (codes u8 [N][K/2], scales u8 [N][K/16], gscale float)."""
    a = np.ascontiguousarray(W, dtype=np.float32)
    N, K = a.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    g = ctypes.c_float(0.0)
    lib().oracle_quantize(_ptr(a, ctypes.c_float), N, K, _ptr(codes, ctypes.c_uint8),
                          _ptr(scales, ctypes.c_uint8), ctypes.byref(g))
    return codes, scales, float(g.value)


# ---- dequant and GEMV ------------------------------------------------------

def dequant(codes: np.ndarray, scales: np.ndarray, gscale: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((N, K), dtype=np.float64)
    lib().oracle_dequant(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                         ctypes.c_float(gscale), N, K, _ptr(out, ctypes.c_double))
    return out


def gemv(codes: np.ndarray, scales: np.ndarray, gscale: float, X_bits: np.ndarray,
         nthreads: int = 0):
    """Return (Y, A), both fp64 [n][N]: Y = X . dequant(W)^T, A = sum |w x|."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    N, K = codes.shape[0], codes.shape[1] * 2
    n = X.shape[0]
    if X.shape[1] != K or scales.shape != (N, K // 16):
        raise ValueError("shape mismatch")
    Y = np.empty((n, N), dtype=np.float64)
    A = np.empty((n, N), dtype=np.float64)
    lib().oracle_gemv(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                      ctypes.c_float(gscale), _ptr(X, ctypes.c_uint16), n, N, K,
                      _ptr(Y, ctypes.c_double), _ptr(A, ctypes.c_double), int(nthreads))
    return Y, A


def gemv_one(codes: np.ndarray, scales: np.ndarray, gscale: float, X_bits: np.ndarray,
             t: int, r: int):
    """One output element (y, A) of the same sum, for sampled checks at full size."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    K = codes.shape[1] * 2
    a = ctypes.c_double(0.0)
    y = lib().oracle_gemv_one(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                              ctypes.c_float(gscale), _ptr(X, ctypes.c_uint16), K, int(t), int(r),
                              ctypes.byref(a))
    return y, a.value


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ---- structural helpers ----------------------------------------------------

def qkv_scatter(Y: np.ndarray, rows, out_off, ldy: int, fill=np.nan) -> np.ndarray:
    """Place the q|k|v row ranges of Y [n][N] at per-projection offsets of a
    token-major output with ``ldy`` elements per token (unwritten slots keep
    ``fill``)."""
    n, N = Y.shape
    if sum(rows) != N:
        raise ValueError("rows must sum to N")
    out = np.full((n, ldy), fill, dtype=Y.dtype)
    start = 0
    for p in range(3):
        out[:, out_off[p]:out_off[p] + rows[p]] = Y[:, start:start + rows[p]]
        start += rows[p]
    return out


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v|: 2^(floor(log2|v|) - 7), floored at 2^-133."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))   # a = f * 2^e with f in [0.5, 1)
    u = np.ldexp(1.0, (e - 1 - 7).astype(np.int64))
    return np.where(a > 0, np.maximum(u, 2.0 ** -133), 2.0 ** -133)


def tolerance(Y_ref: np.ndarray, A_ref: np.ndarray) -> np.ndarray:
    """Acceptance bound per element: 1e-3 * sum|w x| + one bf16 ulp of y."""
    return 1e-3 * np.asarray(A_ref) + ulp_bf16(Y_ref)
