"""Seeded synthetic inputs for the NVFP4 decode-projection workloads.

This module draws random numbers and shapes them into workloads; it holds none
of the method's arithmetic (no NVFP4 encoding or decoding, no GEMV).  Both the
HIP path (through ``bench.py`` and the GPU tests) and the CPU oracle (through
the tests) take their inputs from here.

The shapes are the decode projections the Atlas layer resolver measures at
M=16 (``spark_model::layers`` page, doc comment of ``w4a16_k64_min_k``):
ssm_qkvz 16384x5120, fused attention QKV 14336x5120, ssm_out_proj 5120x6144.
The value distributions follow the stated input recipe: W ~ N(0, 0.02) in fp32,
x ~ N(0, 1) rounded to bf16, optional per-token row scale U(0.5, 2), and an
out_proj variant with 1% all-zero 16-blocks and 1% blocks holding one outlier at
50x the block rms.  Trained checkpoints and real prompts stand in nowhere: all
inputs are synthetic.
"""
from __future__ import annotations

import numpy as np

# (name, N, K) of the workloads; the fused-QKV split is q|k|v = 8192|3072|3072 rows.
SMOKE = ("smoke_1024x1024", 1024, 1024)
QKV = ("fused_qkv_14336x5120", 14336, 5120)
QKVZ = ("ssm_qkvz_16384x5120", 16384, 5120)
OUT_PROJ = ("ssm_out_proj_5120x6144", 5120, 6144)
QKV_ROWS = (8192, 3072, 3072)
N_SWEEP = (1, 2, 3, 4, 8, 16)

WEIGHT_STD = 0.02


def weight_seed(config: int, i: int = 0) -> int:
    return 1000 + 100 * config + i


def act_seed(config: int, n: int) -> int:
    return 2000 + 100 * config + n


def weights_f32(N: int, K: int, seed: int, std: float = WEIGHT_STD) -> np.ndarray:
    """W [N][K] fp32 ~ N(0, std), PCG64 stream of ``seed``."""
    g = np.random.default_rng(seed)
    return (g.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def add_zero_and_outlier_blocks(W: np.ndarray, seed: int, frac_zero: float = 0.01,
                                frac_outlier: float = 0.01, factor: float = 50.0) -> np.ndarray:
    """Copy of W where two disjoint random sets of 16-element K-blocks are edited:
    in the first every element is 0; in the second one uniformly chosen element
    becomes sign(orig) * factor * rms(orig block)."""
    N, K = W.shape
    nb = N * (K // 16)
    g = np.random.default_rng(seed)
    perm = g.permutation(nb)
    nz = int(round(frac_zero * nb))
    no = int(round(frac_outlier * nb))
    zero_blocks = perm[:nz]
    out_blocks = perm[nz:nz + no]
    Wb = W.astype(np.float32).reshape(nb, 16).copy()
    Wb[zero_blocks] = 0.0
    pos = g.integers(0, 16, size=no)
    rms = np.sqrt(np.mean(Wb[out_blocks].astype(np.float64) ** 2, axis=1))
    orig = Wb[out_blocks, pos]
    sign = np.where(orig < 0, -1.0, 1.0)
    Wb[out_blocks, pos] = (sign * factor * rms).astype(np.float32)
    return Wb.reshape(N, K)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activations_bf16(n: int, K: int, seed: int, row_scale: bool = False) -> np.ndarray:
    """X [n][K] as bf16 bit patterns: fp32 N(0,1), optionally times a per-row
    U(0.5, 2) factor, rounded to bf16."""
    g = np.random.default_rng(seed)
    z = g.standard_normal((n, K), dtype=np.float32)
    if row_scale:
        u = g.uniform(0.5, 2.0, size=(n, 1)).astype(np.float32)
        z = (z * u).astype(np.float32)
    return f32_to_bf16_bits(z)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
