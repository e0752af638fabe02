"""Seeded synthetic inputs for the W4A16 linear layer (no quantization arithmetic here).

Shapes and distributions follow the workloads the pages describe for Llama-class
decode and prefill layers: activations ~ N(0, 1) with about 1% of input channels
scaled x20 as salient outliers ("Quantization Paradigms for Edge Inference",
section 3: fewer than 1% of channels carry the salient activations), weights
~ N(0, 0.02^2), and 32 calibration rows drawn like the activations
(same page, section 2 table: AWQ calibrates on about 32 samples).

Both the GPU path and the oracle consume these arrays; this module holds only the
random draws, so it is shared by both without sharing any of the method.
"""
from __future__ import annotations

import numpy as np

OUTLIER_FRACTION = 0.01
OUTLIER_MULT = 20.0
WEIGHT_STD = 0.02
CAL_ROWS = 32

SEED_W, SEED_X, SEED_XCAL, SEED_OUTLIER = 1000, 2000, 3000, 4000


def outlier_channels(k: int, seed: int) -> np.ndarray:
    """round(0.01 K) distinct input channels, sorted."""
    n = int(round(OUTLIER_FRACTION * k))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(k, n, replace=False))


def activations(m: int, k: int, seed: int, outliers: np.ndarray) -> np.ndarray:
    """fp16 [m, k] ~ N(0, 1) with the outlier columns multiplied by 20."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    x[:, outliers] *= OUTLIER_MULT
    return x.astype(np.float16)


def weights(n: int, k: int, seed: int) -> np.ndarray:
    """fp16 [n, k] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(WEIGHT_STD)
    return w.astype(np.float16)


def layer_inputs(config: int, m: int, n: int, k: int, layer: int = 0) -> dict:
    """All inputs of one linear layer: x [m, k], w [n, k], x_cal [32, k], outliers.

    Seeds are fixed per (config index, layer index): W 1000+c+10l, X 2000+c+10l,
    X_cal 3000+c+10l, outlier channels 4000+c (shared by all layers of a config with
    the same K, as the activations of one model share their salient channels).
    """
    off = config + 10 * layer
    outl = outlier_channels(k, SEED_OUTLIER + config)
    return {
        "x": activations(m, k, SEED_X + off, outl),
        "w": weights(n, k, SEED_W + off),
        "x_cal": activations(CAL_ROWS, k, SEED_XCAL + off, outl),
        "outliers": outl,
    }


def signed_permutation(n: int, seed: int, value: float) -> np.ndarray:
    """fp16 [n, n] with one nonzero per row, +-value at a random permuted column."""
    rng = np.random.default_rng(seed)
    cols = rng.permutation(n)
    signs = rng.choice(np.array([-1.0, 1.0]), n)
    w = np.zeros((n, n), dtype=np.float32)
    w[np.arange(n), cols] = signs * value
    return w.astype(np.float16)


def sparse_signs(k: int, count: int, seed: int) -> np.ndarray:
    """fp16 [1, k]: `count` entries of +-1 at random positions, zeros elsewhere."""
    rng = np.random.default_rng(seed)
    x = np.zeros((1, k), dtype=np.float32)
    pos = rng.choice(k, count, replace=False)
    x[0, pos] = rng.choice(np.array([-1.0, 1.0]), count)
    return x.astype(np.float16)
