"""Algorithmic byte and flop counts of the W4A16 linear layer, and MI355X peaks.

Decode is bound by streaming the weights from memory, so the token-rate bound is
memory bandwidth divided by the bytes that must be read per token (edgesiliconlab
?p=2015, section "The Mathematics of Memory Bandwidth Saturation"); prefill is
bound by matrix-core throughput (same section, prefill phase).

Bytes counted for one call y[M, N] = X[M, K] . deq(Wq)^T with group size G:
    codes  N*K/2            (4 bits per weight)
    scales 2*N*K/G          (binary16 per group and output channel)
    zeros  N*K/(2*G)        (4 bits per group and output channel; asymmetric only)
    X      2*M*K, y 2*M*N   (binary16)
    inv_s_c 2*K             (only when the activation rescale is applied in the call)
Flops = 2*M*N*K. Dequantization work and split-K traffic are overhead, not credit.
"""
from __future__ import annotations

FMT_ASYM, FMT_SYM8 = 0, 1

HBM_PEAK_GBS = 8000.0                           # MI355X HBM3E, GB/s (1e9 B/s)
CUS, CLOCK_GHZ = 256, 2.4
MFMA_F16_FLOP_PER_CLK_CU = 4096                 # dense fp16 MFMA
MFMA_F16_PEAK_TFLOPS = CUS * CLOCK_GHZ * MFMA_F16_FLOP_PER_CLK_CU / 1000.0  # 2516.6


def weight_bytes(n: int, k: int, group: int = 128, fmt: int = FMT_ASYM) -> int:
    g = k // group
    b = n * k // 2 + 2 * n * g
    if fmt == FMT_ASYM:
        b += n * g // 2
    return b


def algorithmic_bytes(m: int, n: int, k: int, group: int = 128, fmt: int = FMT_ASYM,
                      with_inv: bool = False) -> int:
    b = weight_bytes(n, k, group, fmt) + 2 * m * k + 2 * m * n
    if with_inv:
        b += 2 * k
    return b


def flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k


def max_tokens_per_s(bandwidth_gbs: float, model_gb: float) -> float:
    """Decode token-rate bound: bandwidth / bytes read per token."""
    return bandwidth_gbs / model_gb


def model_bytes_per_param(group: int = 128, fmt: int = FMT_ASYM) -> float:
    """Stored bytes per weight for the 4-bit group format (codes + metadata)."""
    meta = 2.0 + (0.5 if fmt == FMT_ASYM else 0.0)
    return 0.5 + meta / group
