"""W4A16 AWQ-style weight-only quantized linear layer for MI355X (gfx950).

The compute path lives in the C-ABI library built from ``csrc/`` (HIP kernels for
gfx950); ``awq`` is its thin ctypes binding. Importing the package does not load the
library; the first call into ``awq`` does, and fails loudly if it is not built.
"""
__all__ = ["awq", "synth", "roofline"]
