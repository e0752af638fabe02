"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch each.

Every mutant replaces one piece of the oracle module in place (monkeypatch) with a
wrong variant; the test passes when at least one pin then fails. This shows the pins
are sharp enough that a dropped term, a wrong sign, a wrong rounding rule, a wrong
index or a transposed operand in the oracle cannot go unnoticed.
"""
import numpy as np
import pytest

import oracle
import oracle.awq_oracle as ao
import pins


def _half_up(a):
    return np.floor(np.asarray(a, dtype=np.float64) + 0.5)


def _half_away(a):
    a = np.asarray(a, dtype=np.float64)
    return np.sign(a) * np.floor(np.abs(a) + 0.5)


def _truncate(a):
    return np.trunc(np.asarray(a, dtype=np.float64))


def _fp16_via_f32(a):
    # double rounding through binary32 (a classic mistake)
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def _fp16_no_subnormal(a):
    r = np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)
    return np.where(np.abs(r) < 2.0 ** -14, 0.0, r)


def _dequant_plus_z(q, scales, zeros, group=128):
    q = np.asarray(q, dtype=np.int64)
    s_full = np.repeat(np.asarray(scales, np.float64).T, group, axis=1)
    z_full = np.repeat(np.asarray(zeros, np.int64).T, group, axis=1)
    return ao.fp16_rn((q + z_full) * s_full)


def _dequant_no_zero(q, scales, zeros, group=128):
    q = np.asarray(q, dtype=np.int64)
    s_full = np.repeat(np.asarray(scales, np.float64).T, group, axis=1)
    return ao.fp16_rn(q * s_full)


def _dequant_scale_transposed(q, scales, zeros, group=128):
    q = np.asarray(q, dtype=np.int64)
    s = np.asarray(scales, np.float64)
    z = np.asarray(zeros, np.int64)
    # indexes the scale table as [N, K/G] instead of [K/G, N]
    s_full = np.repeat(s.reshape(s.shape[1], s.shape[0]), group, axis=1)
    z_full = np.repeat(z.T, group, axis=1)
    return ao.fp16_rn((q - z_full) * s_full)


def _dequant_group_off_by_one(q, scales, zeros, group=128):
    q = np.asarray(q, dtype=np.int64)
    s = np.asarray(scales, np.float64)
    z = np.asarray(zeros, np.int64)
    s_full = np.roll(np.repeat(s.T, group, axis=1), 1, axis=1)
    z_full = np.roll(np.repeat(z.T, group, axis=1), 1, axis=1)
    return ao.fp16_rn((q - z_full) * s_full)


def _pack_reversed(codes):
    c = np.asarray(codes, dtype=np.uint64)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    word = np.zeros(c.shape[:-1], dtype=np.uint64)
    for j in range(8):
        word = word + (c[..., j] << np.uint64(4 * (7 - j)))
    return word.astype(np.uint32).view(np.int32)


def _pack_byte_swapped(codes):
    c = np.asarray(codes, dtype=np.uint64)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    word = np.zeros(c.shape[:-1], dtype=np.uint64)
    order = [1, 0, 3, 2, 5, 4, 7, 6]     # high nibble first within each byte
    for j in range(8):
        word = word + (c[..., j] << np.uint64(4 * order[j]))
    return word.astype(np.uint32).view(np.int32)


def _fold_divide(w, s_c):
    return ao.fp16_rn(ao.as_f64(w) / ao.as_f64(s_c)[None, :])


def _fold_rows(w, s_c):
    # scales output rows instead of input columns (a transposed operand)
    w = ao.as_f64(w)
    s = ao.as_f64(s_c)
    n = w.shape[0]
    return ao.fp16_rn(w * np.resize(s, n)[:, None])


def _channel_scale_signed_mean(x_cal, alpha=0.5):
    x = ao.as_f64(x_cal)
    m = x.sum(axis=0) / x.shape[0]
    s = np.where(m > 0, ao.fp16_rn(np.power(np.abs(m), alpha)), 1.0)
    return s, ao.fp16_rn(1.0 / s)


def _channel_scale_no_exponent(x_cal, alpha=0.5):
    x = ao.as_f64(x_cal)
    m = np.abs(x).sum(axis=0) / x.shape[0]
    s = np.where(m > 0, ao.fp16_rn(m), 1.0)
    return s, ao.fp16_rn(1.0 / s)


def _channel_scale_max(x_cal, alpha=0.5):
    x = ao.as_f64(x_cal)
    m = np.abs(x).max(axis=0)
    s = np.where(m > 0, ao.fp16_rn(np.sqrt(m) if alpha == 0.5 else np.power(m, alpha)), 1.0)
    return s, ao.fp16_rn(1.0 / s)


def _matmul_ignores_inv(x, w_d, inv_s_c=None):
    return ao.as_f64(x) @ ao.as_f64(w_d).T


def _matmul_divides_inv(x, w_d, inv_s_c=None):
    x = ao.as_f64(x)
    if inv_s_c is not None:
        x = x / ao.as_f64(inv_s_c)[None, :]
    return x @ ao.as_f64(w_d).T


def _quantize_plain_minmax(w_folded, group=128, fmt=0):
    v = ao._groups(ao.as_f64(w_folded), group)
    if fmt != ao.FMT_ASYM:
        return _orig_quantize(w_folded, group, fmt)
    lo = v.min(axis=2)
    hi = v.max(axis=2)
    s = np.maximum(ao.fp16_rn((hi - lo) / ao.QMAX), ao.SCALE_FLOOR)
    z = np.clip(ao.rint(-lo / s), 0, ao.QMAX)
    q = np.clip(ao.rint(v / s[:, :, None]) + z[:, :, None], 0, ao.QMAX)
    n, k = ao.as_f64(w_folded).shape
    return q.reshape(n, k).astype(np.int64), np.ascontiguousarray(s.T), \
        np.ascontiguousarray(z.T).astype(np.int64)


def _quantize_scale_unrounded(w_folded, group=128, fmt=0):
    saved = ao.fp16_rn
    try:
        ao.fp16_rn = lambda a: np.asarray(a, dtype=np.float64)
        return _orig_quantize(w_folded, group, fmt)
    finally:
        ao.fp16_rn = saved


def _quantize_sym_over_8(w_folded, group=128, fmt=0):
    if fmt != ao.FMT_SYM8:
        return _orig_quantize(w_folded, group, fmt)
    v = ao._groups(ao.as_f64(w_folded), group)
    a = np.abs(v).max(axis=2)
    s = np.maximum(ao.fp16_rn(a / 8.0), ao.SCALE_FLOOR)
    z = np.full_like(s, 8)
    q = np.clip(ao.rint(v / s[:, :, None]) + 8, 0, 15)
    n, k = ao.as_f64(w_folded).shape
    return q.reshape(n, k).astype(np.int64), np.ascontiguousarray(s.T), \
        np.ascontiguousarray(z.T).astype(np.int64)


def _quantize_no_clamp(w_folded, group=128, fmt=0):
    saved = ao.QMAX
    try:
        # codes allowed to 16: the upper clamp goes missing
        ao.QMAX = 16
        return _orig_quantize(w_folded, group, fmt)
    finally:
        ao.QMAX = saved


def _loss_parts(w, x, s_c, group, fmt, fold=True):
    x, w, s = ao.as_f64(x), ao.as_f64(w), ao.as_f64(s_c)
    layer = ao.quantize_layer(w, s if fold else None, group, fmt)
    return x @ w.T, x, s, layer["w_d"]


def _loss_no_sqrt(w, x, s_c, group=128, fmt=0):
    y, x, s, w_d = _loss_parts(w, x, s_c, group, fmt)
    return float(np.sum((y - (x / s[None, :]) @ w_d.T) ** 2))


def _loss_l1(w, x, s_c, group=128, fmt=0):
    y, x, s, w_d = _loss_parts(w, x, s_c, group, fmt)
    return float(np.sum(np.abs(y - (x / s[None, :]) @ w_d.T)))


def _loss_x_times_s(w, x, s_c, group=128, fmt=0):
    y, x, s, w_d = _loss_parts(w, x, s_c, group, fmt)
    return float(np.sqrt(np.sum((y - (x * s[None, :]) @ w_d.T) ** 2)))


def _loss_unfolded_q(w, x, s_c, group=128, fmt=0):
    # the activations are rescaled but the weights are quantized without the fold
    y, x, s, w_d = _loss_parts(w, x, s_c, group, fmt, fold=False)
    return float(np.sqrt(np.sum((y - (x / s[None, :]) @ w_d.T) ** 2)))


def _search_argmax(w, x_cal, group=128, fmt=0, grid=20):
    losses = np.asarray([ao.awq_loss(w, x_cal, ao.channel_scale(x_cal, i / grid)[0], group, fmt)
                         for i in range(grid + 1)])
    return int(np.argmax(losses)) / grid, losses


def _search_fixed_half(w, x_cal, group=128, fmt=0, grid=20):
    # every candidate scored with the same alpha = 1/2 scale
    s, _ = ao.channel_scale(x_cal, 0.5)
    losses = np.asarray([ao.awq_loss(w, x_cal, s, group, fmt) for _ in range(grid + 1)])
    return int(np.argmin(losses)) / grid, losses


_orig_quantize = ao.quantize_rtn

MUTANTS = {
    "rint_half_up": ("rint", _half_up),
    "rint_half_away": ("rint", _half_away),
    "rint_truncate": ("rint", _truncate),
    "fp16_double_rounding_via_f32": ("fp16_rn", _fp16_via_f32),
    "fp16_flush_subnormals": ("fp16_rn", _fp16_no_subnormal),
    "dequant_plus_zero": ("dequant", _dequant_plus_z),
    "dequant_drops_zero": ("dequant", _dequant_no_zero),
    "dequant_scale_transposed": ("dequant", _dequant_scale_transposed),
    "dequant_group_index_shift": ("dequant", _dequant_group_off_by_one),
    "pack_nibbles_reversed": ("_pack_rows", _pack_reversed),
    "pack_nibbles_byte_swapped": ("_pack_rows", _pack_byte_swapped),
    "fold_divides": ("fold", _fold_divide),
    "fold_scales_rows": ("fold", _fold_rows),
    "channel_scale_signed_mean": ("channel_scale", _channel_scale_signed_mean),
    "channel_scale_drops_exponent": ("channel_scale", _channel_scale_no_exponent),
    "channel_scale_uses_max": ("channel_scale", _channel_scale_max),
    "matmul_ignores_rescale": ("matmul_ref", _matmul_ignores_inv),
    "matmul_divides_rescale": ("matmul_ref", _matmul_divides_inv),
    "quantize_minmax_without_zero": ("quantize_rtn", _quantize_plain_minmax),
    "quantize_scale_unrounded": ("quantize_rtn", _quantize_scale_unrounded),
    "quantize_sym_divides_by_8": ("quantize_rtn", _quantize_sym_over_8),
    "quantize_levels_16": ("quantize_rtn", _quantize_no_clamp),
    "loss_without_sqrt": ("awq_loss", _loss_no_sqrt),
    "loss_l1_norm": ("awq_loss", _loss_l1),
    "loss_multiplies_activations": ("awq_loss", _loss_x_times_s),
    "loss_quantizes_unfolded_weights": ("awq_loss", _loss_unfolded_q),
    "search_takes_argmax": ("scale_search", _search_argmax),
    "search_scores_one_scale": ("scale_search", _search_fixed_half),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ao, attr, fn)
    # names re-exported at package level are looked up by the pins through the
    # package object, so patch those too
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed = pins.run_all(oracle)
    assert failed, f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_every_pin():
    assert pins.run_all(oracle) == []
