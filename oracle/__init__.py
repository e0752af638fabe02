"""CPU fp64 oracle of the W4A16 AWQ linear layer.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the benchmark's
CPU-baseline leg. The GPU library shares no code with it.
"""
from .awq_oracle import *  # noqa: F401,F403
from .awq_oracle import (FMT_ASYM, FMT_SYM8, QMAX, SYM_ZERO, SCALE_FLOOR,  # noqa: F401
                         fp16_rn, rint, channel_scale, fold, quantize_rtn, pack_codes,
                         unpack_codes, pack_zeros, unpack_zeros, dequant, dequant_packed,
                         matmul_ref, quantize_layer, awq_loss, scale_search,
                         scales_to_fp16_bits)
