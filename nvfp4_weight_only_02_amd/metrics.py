"""Byte and flop model of the NVFP4 decode projection (host arithmetic only).

Weights cost 9/16 byte each (a 4-bit E2M1 code plus one E4M3 byte per 16
weights); activations and outputs are bf16.  The spark_model::layers page
(doc comment of K64_N64_MAX_WIDE_CTAS) decomposes its out_proj replay into
bytes moved at 95.6% of a 229.6 GB/s ceiling in 87.2 us; that figure matches
this model for N=5120, K=6144 and 64 token rows to 0.02%.
"""

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published peak
BF16_DENSE_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published peak


def weight_bytes(N: int, K: int) -> int:
    return N * K // 2 + N * K // 16


def algorithmic_bytes(n: int, N: int, K: int) -> int:
    """Bytes one call must move at least: weights once, X in, Y out."""
    return weight_bytes(N, K) + 2 * n * K + 2 * n * N


def flops(n: int, N: int, K: int) -> int:
    return 2 * n * N * K
