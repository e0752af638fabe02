"""The benchmark's byte/flop model against the pages' printed figures and closed forms."""
import pytest

import pins
from bit_weight_only_w4a16_amd import roofline as rl


def test_bandwidth_bound_example():
    g = pins.load_golden("bandwidth_model.txt")
    bw = float(g["bandwidth_gbs"])
    for fmt in ("fp16", "awq"):
        got = rl.max_tokens_per_s(bw, float(g[f"{fmt}.model_gb"]))
        printed = float(g[f"{fmt}.max_tok_s"])
        assert printed <= got < printed + 0.1


def test_footprint_70b():
    g = pins.load_golden("footprint.txt")
    p = float(g["params"])
    assert round(p * 2 / 1e9) == int(g["fp16.gb"])
    assert round(p * 0.5 / 1e9) == int(g["int4_codes.gb"])
    assert round(p * rl.model_bytes_per_param(128, rl.FMT_ASYM) / 1e9) == int(g["awq_group128.gb"])


def test_closed_form_bytes():
    # 4096 -> 4096 at M = 1: codes 8 388 608 + scales 262 144 + zeros 65 536 + x 8192 + y 8192
    assert rl.algorithmic_bytes(1, 4096, 4096) == 8_732_672
    assert rl.algorithmic_bytes(1, 11008, 4096) == 23_455_232
    assert rl.algorithmic_bytes(1, 4096, 11008) == 23_455_232
    assert rl.weight_bytes(4096, 4096, 128, rl.FMT_SYM8) == 8_388_608 + 262_144
    assert rl.algorithmic_bytes(1, 4096, 4096, with_inv=True) == 8_732_672 + 8192
    assert rl.flops(2048, 6144, 4096) == 2 * 2048 * 6144 * 4096
    # fp16 / int4 bytes ratio at M = 1 tends to 2 / (0.5 + 2.5/128) = 3.85
    assert rl.model_bytes_per_param() == pytest.approx(0.51953125)
    assert 2 / rl.model_bytes_per_param() == pytest.approx(3.8496, abs=1e-4)


def test_peaks():
    assert rl.MFMA_F16_PEAK_TFLOPS == pytest.approx(2516.58, abs=0.01)
    assert rl.HBM_PEAK_GBS == 8000.0
