"""Plain CPU fp64 oracle for the W4A16 (AWQ-style) weight-only quantized linear layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module. The GPU library never calls it, links it or
reads values it produced; the two share no code.

What it computes, in the order the pages give it:

  1. a per-input-channel scale from calibration activations
     ("Quantization Paradigms for Edge Inference", section 3 "The Math Behind
     Activation-Aware Protection (AWQ)": salient channels are found from activation
     magnitudes under a calibration distribution);
  2. the fold W' = W diag(s), X' = diag(s)^-1 X (same section, first equation);
  3. round-to-nearest uniform 4-bit quantization of each group of G weights along K
     with one scale and one zero point per group (edgesiliconlab ?p=2015, section
     "What Is the Core Difference Between AWQ and GPTQ Quantization?" for RTN on the
     scaled matrix; "The Ultimate Guide to Quantized LLMs: GPTQ", section
     "Understanding Quantized Model Compression" for blockwise scales and zero points);
  4. packing of the 4-bit codes several to a machine word (edgesiliconlab ?p=2015,
     section "Kernel Execution: Marlin vs. ExLlamaV2 INT4 GEMM Micro-Architecture",
     item 3: 4-bit values sit side by side in a word and are recovered by shift and
     mask);
  5. dequantization deq(q) = (q - z) * s, and the product y = X' . deq(Wq)^T, which
     stands in for X . W^T.

Everything is float64 numpy; a library primitive (numpy's float64 -> float16
conversion, numpy's matmul) is used as a single step where noted. No blocking,
fusion or reordering beyond the definitions.

Readings where the pages leave a step open (each is listed again in the design
notes): scale of an asymmetric group = (max(v,0) - min(v,0)) / 15 rounded to
binary16 and floored at 2^-24; zero = rint(-min(v,0)/s) clamped to [0,15];
code = rint(v/s) + zero clamped to [0,15]; rint is round-half-to-even; the
symmetric variant uses scale = max|v| / 7 and a fixed zero of 8; the channel scale
is s_c = (mean_r |X_cal[r,k]|)^alpha rounded to binary16 (1 where the mean is 0),
with no normalisation; inv_s_c = binary16(1 / s_c).

Parity status: the rules above are pinned by hand-worked examples, closed forms and
brute force in the CPU tests; no page prints a quantized value, so the choice of
scale rule itself is a reading, not something the pages pin.
"""
from __future__ import annotations

import numpy as np

FMT_ASYM = 0   # asymmetric: per-group fp16 scale and uint4 zero point
FMT_SYM8 = 1   # symmetric "GPTQ-style": per-group fp16 scale, zero fixed at 8

QMAX = 15                 # 4-bit codes 0..15
SYM_ZERO = 8
SCALE_FLOOR = 2.0 ** -24  # smallest positive binary16 (subnormal)


# --------------------------------------------------------------------------- helpers

def fp16_rn(a) -> np.ndarray:
    """Round float64 values to the nearest IEEE-754 binary16 value, ties to even,
    subnormals kept, overflow to +-inf; returned as float64.

    One library step: numpy's direct float64 -> float16 conversion. The CPU tests pin
    it against the binary16 definition on every finite value and every midpoint.
    """
    with np.errstate(over="ignore"):  # overflow to +-inf is the defined result
        return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def rint(a) -> np.ndarray:
    """Round to the nearest integer, ties to even (the 'nearest' of round-to-nearest)."""
    return np.rint(np.asarray(a, dtype=np.float64))


def as_f64(a) -> np.ndarray:
    """Exact float64 copy of a float16 (or already float64) array."""
    return np.asarray(a).astype(np.float64)


# ----------------------------------------------------------------- 1. channel scale

def channel_scale(x_cal, alpha: float = 0.5):
    """Per-input-channel AWQ scale from calibration rows.

    "Quantization Paradigms for Edge Inference", section 3: the salient channels are
    identified from activation magnitudes over a calibration distribution. Here
    m_k = mean over rows of |X_cal[r, k]| (the sum of binary16 magnitudes is exact in
    float64 for up to 8192 rows), s_c[k] = binary16(m_k ** alpha), or 1 where m_k = 0.
    alpha = 0.5 uses the correctly rounded square root.

    Returns (s_c, inv_s_c), both float64 arrays holding binary16 values;
    inv_s_c = binary16(1 / s_c).
    """
    x = as_f64(x_cal)
    if x.ndim != 2:
        raise ValueError("x_cal must be [rows, K]")
    m = np.abs(x).sum(axis=0) / x.shape[0]
    if alpha == 0.5:
        p = np.sqrt(m)
    else:
        p = np.power(m, alpha)
    s = np.where(m > 0, fp16_rn(p), 1.0)
    inv = fp16_rn(1.0 / s)
    return s, inv


# ------------------------------------------------------------------------- 2. fold

def fold(w, s_c) -> np.ndarray:
    """W' = W diag(s_c): scale input channel k (column k of W[N, K]) by s_c[k].

    "Quantization Paradigms for Edge Inference", section 3, first equation. The
    product of two binary16 values is exact in float64, so W' = binary16(W * s_c)
    carries exactly one rounding.
    """
    w = as_f64(w)
    s = as_f64(s_c)
    return fp16_rn(w * s[None, :])


# ------------------------------------------------------------------- 3. quantize

def _groups(w: np.ndarray, group: int) -> np.ndarray:
    n, k = w.shape
    if k % group != 0:
        raise ValueError("K must be a multiple of the group size")
    return w.reshape(n, k // group, group)


def quantize_rtn(w_folded, group: int = 128, fmt: int = FMT_ASYM):
    """Round-to-nearest 4-bit group quantization of W'[N, K] along K.

    One scale and one zero point per (output row n, group g of `group` consecutive
    input channels): "The Ultimate Guide to Quantized LLMs: GPTQ", section
    "Understanding Quantized Model Compression"; RTN on the scaled matrix:
    edgesiliconlab ?p=2015, section "What Is the Core Difference Between AWQ and
    GPTQ Quantization?".

    Asymmetric (fmt=0), for each group v:
        lo = min(min v, 0), hi = max(max v, 0)
        s  = max(binary16((hi - lo) / 15), 2^-24)
        z  = clamp(rint(-lo / s), 0, 15)
        q  = clamp(rint(v / s) + z, 0, 15)
    Symmetric (fmt=1): s = max(binary16(max|v| / 7), 2^-24), z = 8,
        q = clamp(rint(v / s) + 8, 0, 15).

    Returns q int64 [N, K], scales float64 [K/group, N] (binary16 values),
    zeros int64 [K/group, N].
    """
    v = _groups(as_f64(w_folded), group)                     # [N, Gs, group]
    if fmt == FMT_ASYM:
        lo = np.minimum(v.min(axis=2), 0.0)                  # [N, Gs]
        hi = np.maximum(v.max(axis=2), 0.0)
        s = np.maximum(fp16_rn((hi - lo) / QMAX), SCALE_FLOOR)
        z = np.clip(rint(-lo / s), 0, QMAX)
    elif fmt == FMT_SYM8:
        a = np.abs(v).max(axis=2)
        s = np.maximum(fp16_rn(a / 7.0), SCALE_FLOOR)
        z = np.full_like(s, SYM_ZERO)
    else:
        raise ValueError("fmt must be 0 (asymmetric) or 1 (symmetric, zero 8)")
    q = np.clip(rint(v / s[:, :, None]) + z[:, :, None], 0, QMAX)
    n, k = as_f64(w_folded).shape
    return (q.reshape(n, k).astype(np.int64),
            np.ascontiguousarray(s.T),
            np.ascontiguousarray(z.T).astype(np.int64))


# ------------------------------------------------------------------------ 4. pack

def _pack_rows(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes along the last axis, 8 per 32-bit word, element 8w+j in
    bits 4j..4j+3 of word w; returned as two's-complement int32."""
    c = np.asarray(codes, dtype=np.uint64)
    if c.shape[-1] % 8 != 0:
        raise ValueError("last axis must be a multiple of 8")
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    word = np.zeros(c.shape[:-1], dtype=np.uint64)
    for j in range(8):
        word = word + (c[..., j] << np.uint64(4 * j))
    return word.astype(np.uint32).view(np.int32)


def _unpack_rows(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words).view(np.uint32).astype(np.uint64)
    out = np.empty(w.shape + (8,), dtype=np.int64)
    for j in range(8):
        out[..., j] = ((w >> np.uint64(4 * j)) & np.uint64(0xF)).astype(np.int64)
    return out.reshape(w.shape[:-1] + (w.shape[-1] * 8,))


def pack_codes(q) -> np.ndarray:
    """qweight int32 [N, K/8] from codes [N, K] (nibbles along K)."""
    return _pack_rows(q)


def unpack_codes(qweight) -> np.ndarray:
    return _unpack_rows(qweight)


def pack_zeros(z) -> np.ndarray:
    """qzeros int32 [K/G, N/8] from zero points [K/G, N] (nibbles along N)."""
    return _pack_rows(z)


def unpack_zeros(qzeros) -> np.ndarray:
    return _unpack_rows(qzeros)


def scales_to_fp16_bits(scales) -> np.ndarray:
    """binary16 bit patterns (uint16) of a float64 array of binary16 values."""
    return np.asarray(scales, dtype=np.float64).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------- 5. dequant

def dequant(q, scales, zeros, group: int = 128) -> np.ndarray:
    """W_d[n, k] = binary16((q[n, k] - z[g, n]) * s[g, n]) with g = k // group.

    The float64 product of a small integer and a binary16 value is exact, so there is
    one rounding. This is the bit-exact target for every dequantizing kernel.
    """
    q = np.asarray(q, dtype=np.int64)
    n, k = q.shape
    s = as_f64(scales)                    # [K/G, N]
    z = np.asarray(zeros, dtype=np.int64)  # [K/G, N]
    s_full = np.repeat(s.T, group, axis=1)  # [N, K]
    z_full = np.repeat(z.T, group, axis=1)
    return fp16_rn((q - z_full).astype(np.float64) * s_full)


def matmul_ref(x, w_d, inv_s_c=None) -> np.ndarray:
    """y[m, n] = sum_k (X[m, k] * inv_s_c[k]) * W_d[n, k], all float64.

    With inv_s_c None, X is taken as already rescaled (X'). One library step: numpy
    matmul in float64.
    """
    x = as_f64(x)
    if inv_s_c is not None:
        x = x * as_f64(inv_s_c)[None, :]
    return x @ as_f64(w_d).T


# --------------------------------------------------------- whole offline pipeline

def quantize_layer(w, s_c=None, group: int = 128, fmt: int = FMT_ASYM) -> dict:
    """Fold (if s_c given), quantize and pack one weight matrix W[N, K].

    Returns a dict with the canonical packed tensors and the unpacked intermediates:
    w_folded, q, scales, zeros, qweight, qzeros (None for the symmetric format),
    scales_bits (uint16 binary16 patterns), w_d (dequantized, float64).
    """
    wf = fold(w, s_c) if s_c is not None else as_f64(w)
    q, s, z = quantize_rtn(wf, group, fmt)
    return {
        "w_folded": wf,
        "q": q,
        "scales": s,
        "zeros": z,
        "qweight": pack_codes(q),
        "qzeros": pack_zeros(z) if fmt == FMT_ASYM else None,
        "scales_bits": scales_to_fp16_bits(s),
        "w_d": dequant(q, s, z, group),
    }


def dequant_packed(qweight, scales, qzeros, group: int = 128, fmt: int = FMT_ASYM):
    """Dequantize from the canonical packed tensors (qzeros None for symmetric)."""
    q = unpack_codes(qweight)
    s = as_f64(scales)
    if fmt == FMT_ASYM:
        z = unpack_zeros(qzeros)
    else:
        z = np.full(s.shape, SYM_ZERO, dtype=np.int64)
    return dequant(q, s, z, group)


# ----------------------------------------------------- objective of the scale search

def awq_loss(w, x, s_c, group: int = 128, fmt: int = FMT_ASYM) -> float:
    """|| X W^T - (X diag(s)^-1) Q(W diag(s))^T ||_2 (Frobenius), float64.

    "Quantization Paradigms for Edge Inference", section 3, second equation, written
    in the row convention y = X W^T. Q is the fold + RTN + dequant of this module;
    diag(s)^-1 is applied exactly in float64.
    """
    x = as_f64(x)
    w = as_f64(w)
    s = as_f64(s_c)
    layer = quantize_layer(w, s, group, fmt)
    y_true = x @ w.T
    y_q = (x / s[None, :]) @ layer["w_d"].T
    return float(np.sqrt(np.sum((y_true - y_q) ** 2)))


def scale_search(w, x_cal, group: int = 128, fmt: int = FMT_ASYM, grid: int = 20):
    """Grid search of the exponent alpha in s = mean|X_cal|^alpha minimising awq_loss
    on the calibration rows ("Quantization Paradigms for Edge Inference", section 3,
    second equation: the scale is searched to minimise the output error). The pages
    do not fix the search space; alpha in {0, 1/grid, ..., 1} is this oracle's
    reading. Ties keep the smallest alpha. Returns (best_alpha, losses[grid+1]).
    """
    losses = []
    for i in range(grid + 1):
        a = i / grid
        s, _ = channel_scale(x_cal, a)
        losses.append(awq_loss(w, x_cal, s, group, fmt))
    losses = np.asarray(losses)
    best = int(np.argmin(losses))
    return best / grid, losses
