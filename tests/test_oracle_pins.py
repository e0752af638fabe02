"""The CPU oracle against hand-worked examples, closed forms and brute force."""
import numpy as np
import pytest

import oracle
import pins
from bit_weight_only_w4a16_amd import synth


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)


def test_awq_beats_rtn_on_outlier_activations():
    """Quality property of the fold (statistical, not parity): on the 1%-outlier
    synthetic layer the scaled quantization has lower output error than plain RTN
    against the unquantized product, over 64 held-out rows, in most seeds."""
    wins = 0
    for seed in range(6):
        d = synth.layer_inputs(seed, 64, 512, 512)
        x = oracle.as_f64(d["x"])
        w = oracle.as_f64(d["w"])
        y_true = x @ w.T
        s_c, inv = oracle.channel_scale(d["x_cal"], 0.5)
        awq = oracle.quantize_layer(w, s_c, 128, oracle.FMT_ASYM)
        rtn = oracle.quantize_layer(w, None, 128, oracle.FMT_ASYM)
        e_awq = np.linalg.norm(oracle.matmul_ref(x, awq["w_d"], inv) - y_true)
        e_rtn = np.linalg.norm(oracle.matmul_ref(x, rtn["w_d"]) - y_true)
        wins += e_awq < e_rtn
    assert wins >= 5


def test_loss_objective_prefers_scaling():
    """The search objective L(s) is lower at alpha = 0.5 than at alpha = 0 (no
    scaling) on the calibration rows of the outlier layer."""
    d = synth.layer_inputs(0, 1, 512, 512)
    s_half, _ = oracle.channel_scale(d["x_cal"], 0.5)
    ones = np.ones(512)
    l_half = oracle.awq_loss(d["w"], d["x_cal"], s_half)
    l_one = oracle.awq_loss(d["w"], d["x_cal"], ones)
    assert l_half < l_one
    best, losses = oracle.scale_search(d["w"], d["x_cal"], grid=4)
    assert losses.shape == (5,) and losses[int(best * 4)] == losses.min()
    assert best > 0


def test_zero_alpha_is_plain_rtn():
    d = synth.layer_inputs(0, 1, 256, 256)
    s0, inv0 = oracle.channel_scale(d["x_cal"], 0.0)
    a = oracle.quantize_layer(d["w"], s0, 128)
    b = oracle.quantize_layer(d["w"], None, 128)
    assert np.all(s0 == 1.0) and np.all(inv0 == 1.0)
    assert np.array_equal(a["qweight"], b["qweight"])
    assert np.array_equal(a["scales"], b["scales"])
