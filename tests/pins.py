"""Pins of the CPU oracle against facts fixed outside it.

Each pin takes the oracle module and raises AssertionError when the oracle disagrees
with a hand-worked example, a closed form, a special case or brute force. The same
pins run against deliberately broken copies of the oracle in test_oracle_mutations
to show that each plausible mistake is caught by at least one of them.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (p.strip() for p in line.split("=", 1))
            out[key] = val
    return out


def _nums(s: str, dtype=float):
    return np.array([dtype(t) for t in s.split()])


# ------------------------------------------------------------------ binary16 rounding

def _f16_value(bits: np.ndarray) -> np.ndarray:
    """Value of binary16 bit patterns from the format definition (sign, 5-bit biased
    exponent, 10-bit fraction), computed with integer arithmetic and ldexp."""
    bits = bits.astype(np.int64)
    sign = np.where(bits >> 15, -1.0, 1.0)
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -24),
                   np.ldexp((f + 1024).astype(np.float64), (e - 25).astype(np.int64)))
    return sign * mag


def pin_fp16_exhaustive(o):
    """Every finite binary16 value round-trips; every midpoint between neighbours
    rounds to the neighbour with an even fraction; one float64 ulp either side of a
    midpoint rounds to the nearer neighbour; overflow goes to infinity."""
    bits = np.arange(0, 0x7C00, dtype=np.int64)           # +0 .. max finite
    vals = _f16_value(bits)
    assert np.array_equal(o.fp16_rn(vals), vals)
    assert np.array_equal(o.fp16_rn(-vals), -vals)
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2                                     # exact in float64
    even = np.where((bits[:-1] & 1) == 0, lo, hi)
    assert np.array_equal(o.fp16_rn(mid), even)
    assert np.array_equal(o.fp16_rn(-mid), -even)
    assert np.array_equal(o.fp16_rn(np.nextafter(mid, -np.inf)), lo)
    assert np.array_equal(o.fp16_rn(np.nextafter(mid, np.inf)), hi)
    # above the largest finite value: 65504 + half an ulp (16) ties to the even
    # neighbour, which is the overflow to infinity
    assert o.fp16_rn(np.array([65519.99]))[0] == 65504.0
    assert np.isinf(o.fp16_rn(np.array([65520.0]))[0])
    assert o.fp16_rn(np.array([2.0 ** -25]))[0] == 0.0      # tie below the subnormal
    assert o.fp16_rn(np.array([2.0 ** -25 * 1.5]))[0] == 2.0 ** -24


# ---------------------------------------------------------------- hand-worked 2x8

def pin_hand_dequant(o):
    g = load_golden("hand_2x8.txt")
    q = np.stack([_nums(g["row0.q"], int), _nums(g["row1.q"], int)])
    s = np.array([[float(g["row0.s"]), float(g["row1.s"])]])          # [1 group, 2 n]
    z = np.array([[int(g["row0.z"]), int(g["row1.z"])]])
    w_d = o.dequant(q, s, z, group=8)
    assert np.array_equal(w_d[0], _nums(g["row0.deq"]))
    assert np.array_equal(w_d[1], _nums(g["row1.deq"]))


def pin_hand_pack(o):
    g = load_golden("hand_2x8.txt")
    q = np.stack([_nums(g["row0.q"], int), _nums(g["row1.q"], int)])
    words = o.pack_codes(q)
    assert words.dtype == np.int32 and words.shape == (2, 1)
    assert words[0, 0] == int(g["row0.word_int32"])
    assert words[1, 0] == int(g["row1.word_int32"])
    assert words.view(np.uint32)[0, 0] == int(g["row0.word_hex"], 16)
    assert words.view(np.uint32)[1, 0] == int(g["row1.word_hex"], 16)
    assert np.array_equal(o.unpack_codes(words), q)
    z = _nums(g["zeros8.z"], int)[None, :]
    zw = o.pack_zeros(z)
    assert zw.shape == (1, 1) and zw.view(np.uint32)[0, 0] == int(g["zeros8.word_hex"], 16)
    assert np.array_equal(o.unpack_zeros(zw), z)


def pin_hand_product(o):
    g = load_golden("hand_2x8.txt")
    w_d = np.stack([_nums(g["row0.deq"]), _nums(g["row1.deq"])])
    y = o.matmul_ref(np.ones((1, 8)), w_d)
    assert np.array_equal(y[0], _nums(g["x_ones.y"]))
    # the activation rescale multiplies column k of X by inv_s_c[k]
    inv = np.array([2.0, 1, 1, 1, 1, 1, 1, 0.5])
    y2 = o.matmul_ref(np.ones((1, 8)), w_d, inv)
    assert np.array_equal(y2[0], np.array([18 - 1.5 - 3.0, -0.5 + 1.75 - 0.375]))


def pin_hand_requantize(o):
    """Re-quantizing the dequantized hand rows returns the same scale, zero, codes."""
    g = load_golden("hand_2x8.txt")
    w_d = np.stack([_nums(g["row0.deq"]), _nums(g["row1.deq"])])
    q, s, z = o.quantize_rtn(w_d, group=8, fmt=o.FMT_ASYM)
    assert np.array_equal(s[0], [0.5, 0.25])
    # row 1 has no code 0: its minimum is -2 = (0 - 8) * 0.25, its maximum 1.75,
    # so the range is 3.75 -> scale 0.25 and zero rint(2 / 0.25) = 8
    assert np.array_equal(z[0], [3, 8])
    assert np.array_equal(q[0], _nums(g["row0.q"], int))
    assert np.array_equal(q[1], _nums(g["row1.q"], int))


# --------------------------------------------------------------------- tie-break

def pin_tie_break(o):
    g = load_golden("tie_break.txt")
    v = _nums(g["group.v"])[None, :]
    q, s, z = o.quantize_rtn(v, group=8, fmt=o.FMT_ASYM)
    assert s[0, 0] == float(g["expect.s"]) and z[0, 0] == int(g["expect.z"])
    assert np.array_equal(q[0], _nums(g["expect.q"], int))
    assert not np.array_equal(q[0], _nums(g["half_up.q"], int))
    assert not np.array_equal(q[0], _nums(g["half_away.q"], int))


# ------------------------------------------------------------- on-grid reproduction

def pin_on_grid_exact(o, seed=7, n=16, k=512, group=128):
    """W built on the 4-bit grid, W = (q - z) s with s of at most 7 significant bits
    and codes 0 and 15 present in every group: min-max recovers s and z exactly,
    the codes come back unchanged and the dequantized W equals W bit for bit."""
    rng = np.random.default_rng(seed)
    gs = k // group
    mant = rng.integers(64, 128, size=(gs, n))                   # 7 significant bits
    expo = rng.integers(-14, -6, size=(gs, n))
    s = np.ldexp(mant.astype(np.float64), expo)                  # exact binary16
    z = rng.integers(0, 16, size=(gs, n))
    q = rng.integers(0, 16, size=(n, k))
    for gi in range(gs):                                         # force 0 and 15
        q[:, gi * group] = 0
        q[:, gi * group + 1] = 15
    s_full = np.repeat(s.T, group, axis=1)
    z_full = np.repeat(z.T, group, axis=1)
    w = (q - z_full) * s_full
    assert np.array_equal(o.fp16_rn(w), w)                       # on the binary16 grid
    q2, s2, z2 = o.quantize_rtn(w, group, o.FMT_ASYM)
    assert np.array_equal(s2, s)
    assert np.array_equal(z2, z)
    assert np.array_equal(q2, q)
    assert np.array_equal(o.dequant(q2, s2, z2, group), w)
    layer = o.quantize_layer(w, None, group, o.FMT_ASYM)
    assert np.array_equal(o.dequant_packed(layer["qweight"], layer["scales"],
                                           layer["qzeros"], group, o.FMT_ASYM), w)


def pin_sym_on_grid(o, seed=8, n=8, k=256, group=128):
    """Symmetric format: W = (q - 8) s with codes 1 and 15 in every group (so
    max|W| = 7 s) is recovered exactly; code 0 is never produced for such W."""
    rng = np.random.default_rng(seed)
    gs = k // group
    s = np.ldexp(rng.integers(64, 128, size=(gs, n)).astype(np.float64),
                 rng.integers(-14, -6, size=(gs, n)))
    q = rng.integers(1, 16, size=(n, k))
    for gi in range(gs):
        q[:, gi * group] = 1
        q[:, gi * group + 5] = 15
    w = (q - 8) * np.repeat(s.T, group, axis=1)
    q2, s2, z2 = o.quantize_rtn(w, group, o.FMT_SYM8)
    assert np.array_equal(s2, s) and np.all(z2 == 8) and np.array_equal(q2, q)
    layer = o.quantize_layer(w, None, group, o.FMT_SYM8)
    assert layer["qzeros"] is None
    assert np.array_equal(o.dequant_packed(layer["qweight"], layer["scales"], None,
                                           group, o.FMT_SYM8), w)


# -------------------------------------------------------------- degenerate groups

def pin_degenerate_groups(o):
    """All-zero group: scale 2^-24, zero 0, codes 0, dequant 0. A constant positive
    group c: range [0, c], codes 15, dequant within half a step of c. A constant
    negative group -c: zero 15, codes 0."""
    group = 16
    w = np.zeros((3, group))
    w[1, :] = 0.75
    w[2, :] = -0.75
    q, s, z = o.quantize_rtn(w, group, o.FMT_ASYM)
    assert s[0, 0] == 2.0 ** -24 and z[0, 0] == 0 and np.all(q[0] == 0)
    assert s[0, 1] == o.fp16_rn(0.75 / 15) and z[0, 1] == 0 and np.all(q[1] == 15)
    assert s[0, 2] == o.fp16_rn(0.75 / 15) and z[0, 2] == 15 and np.all(q[2] == 0)
    w_d = o.dequant(q, s, z, group)
    assert np.all(w_d[0] == 0)
    assert np.all(np.abs(w_d[1] - 0.75) <= s[0, 1] / 2)
    assert np.all(np.abs(w_d[2] + 0.75) <= s[0, 2] / 2)
    qs, ss, zs = o.quantize_rtn(w, group, o.FMT_SYM8)
    assert ss[0, 0] == 2.0 ** -24 and np.all(qs[0] == 8)
    assert np.all(qs[1] == 15) and np.all(qs[2] == 1)


# ---------------------------------------------------------------- RTN error bound

def pin_rtn_error_bound(o, seed=11, n=64, k=1024, group=128):
    """For random weights, every code not at a clamp satisfies |v/s - (q - z)| <= 1/2
    (round to nearest), the group minimum gets code 0 (asymmetric), clamps are rare,
    and |W' - W_d| <= s/2 + half a binary16 ulp of W_d."""
    rng = np.random.default_rng(seed)
    w = o.fp16_rn(rng.standard_normal((n, k)) * 0.02)
    for fmt in (o.FMT_ASYM, o.FMT_SYM8):
        q, s, z = o.quantize_rtn(w, group, fmt)
        s_full = np.repeat(s.T, group, axis=1)
        z_full = np.repeat(z.T, group, axis=1)
        r = w / s_full - (q - z_full)
        inner = (q > 0) & (q < 15)
        assert np.all(np.abs(r[inner]) <= 0.5)
        # every group's minimum and maximum sit at codes 0 and 15: 2 / group of them
        assert np.mean(~inner) < max(0.05, 2.0 / group + 0.03)
        w_d = o.dequant(q, s, z, group)
        ulp_half = np.ldexp(1.0, np.frexp(np.abs(w_d) + 2.0 ** -24)[1] - 12)
        assert np.all(np.abs(w - w_d) <= 0.5 * s_full * (1 + 2.0 ** -5) + ulp_half)
        if fmt == o.FMT_ASYM:
            gmin = np.argmin(w.reshape(n, k // group, group), axis=2)
            qg = q.reshape(n, k // group, group)
            assert np.all(np.take_along_axis(qg, gmin[..., None], 2) == 0)


def pin_small_groups(o):
    """The on-grid recoveries (both formats) and the rounding bound again with groups
    of 32 and 64 channels, four and two groups per 128 channels."""
    for group in (32, 64):
        pin_on_grid_exact(o, seed=17 + group, n=8, k=256, group=group)
        pin_sym_on_grid(o, seed=18 + group, n=8, k=256, group=group)
        pin_rtn_error_bound(o, seed=19 + group, n=16, k=512, group=group)


# ------------------------------------------------------------------------ fold

def pin_fold_invariance(o, seed=3):
    """(W diag(s)) (diag(s)^-1 X) = W X: exact for power-of-two s (no rounding in the
    fold), and within 1e-12 relative for general s before any rounding."""
    rng = np.random.default_rng(seed)
    n, k, m = 24, 64, 5
    w = o.fp16_rn(rng.standard_normal((n, k)) * 0.02)
    x = o.fp16_rn(rng.standard_normal((m, k)))
    s = np.ldexp(1.0, rng.integers(0, 4, size=k))          # >= 1: no binary16 bit lost
    wf = o.fold(w, s)
    assert np.array_equal(wf, w * s[None, :])
    assert np.array_equal((x / s[None, :]) @ wf.T, x @ w.T)
    s2 = rng.uniform(0.3, 3.0, size=k)
    lhs = (x / s2[None, :]) @ (w * s2[None, :]).T
    assert np.max(np.abs(lhs - x @ w.T)) <= 1e-12 * np.max(np.abs(x @ w.T))


# ---------------------------------------------------------------- channel scale

def pin_channel_scale(o):
    """Columns with constant |x| = c (alternating signs) give s = binary16(sqrt(c));
    a zero column gives 1; inv = binary16(1/s); alpha = 1 gives binary16(c) and
    alpha = 0 gives 1."""
    cs = np.array([4.0, 0.25, 2.0, 0.0, 9.0, 0.1])
    rows = 32
    sign = np.where(np.arange(rows) % 2 == 0, 1.0, -1.0)[:, None]
    x = o.fp16_rn(sign * cs[None, :])
    c16 = np.abs(x[0])
    s, inv = o.channel_scale(x, 0.5)
    expect = np.where(c16 > 0, o.fp16_rn(np.sqrt(c16)), 1.0)
    assert np.array_equal(s, expect)
    assert np.array_equal(s[[0, 1, 3, 4]], [2.0, 0.5, 1.0, 3.0])
    assert np.array_equal(inv, o.fp16_rn(1.0 / expect))
    s1, _ = o.channel_scale(x, 1.0)
    assert np.array_equal(s1, np.where(c16 > 0, c16, 1.0))
    s0, _ = o.channel_scale(x, 0.0)
    assert np.all(s0 == 1.0)
    # mean over rows, not a single row
    x2 = np.zeros((4, 1))
    x2[:, 0] = [1.0, 3.0, 0.0, 0.0]
    assert o.channel_scale(x2, 1.0)[0][0] == 1.0


# ------------------------------------------------------------------- brute force

def _brute_quantize(vals, fmt):
    """Scalar transcription of the group rule for one group (pure Python)."""
    import math
    if fmt == 0:
        lo = min(min(vals), 0.0)
        hi = max(max(vals), 0.0)
        s = float(np.float16((hi - lo) / 15.0))
        s = max(s, 2.0 ** -24)
        z = min(max(round(-lo / s), 0), 15)          # Python round = half to even
    else:
        s = max(float(np.float16(max(abs(v) for v in vals) / 7.0)), 2.0 ** -24)
        z = 8
    qs = [min(max(round(v / s) + z, 0), 15) for v in vals]
    assert all(math.isfinite(v) for v in vals)
    return qs, s, z


def pin_brute_force(o, seed=5):
    """Pure-Python loops on tiny shapes: quantize (per group), pack (per nibble),
    dequantize and the triple-loop product, including the fold and rescale."""
    rng = np.random.default_rng(seed)
    for (m, n, k, group, fmt) in [(1, 8, 16, 8, 0), (3, 16, 32, 16, 0), (2, 8, 32, 8, 1)]:
        w = o.fp16_rn(rng.standard_normal((n, k)) * 0.05)
        x = o.fp16_rn(rng.standard_normal((m, k)))
        x_cal = o.fp16_rn(rng.standard_normal((4, k)) * 2)
        s_c, inv = o.channel_scale(x_cal, 0.5)
        layer = o.quantize_layer(w, s_c, group, fmt)
        wf = [[float(np.float16(float(w[i, j]) * float(s_c[j]))) for j in range(k)]
              for i in range(n)]
        assert np.array_equal(layer["w_folded"], np.array(wf))
        for i in range(n):
            for gi in range(k // group):
                qs, s, z = _brute_quantize(wf[i][gi * group:(gi + 1) * group], fmt)
                assert list(layer["q"][i, gi * group:(gi + 1) * group]) == qs
                assert layer["scales"][gi, i] == s and layer["zeros"][gi, i] == z
        for i in range(n):
            for wi in range(k // 8):
                word = 0
                for j in range(8):
                    word |= int(layer["q"][i, 8 * wi + j]) << (4 * j)
                assert int(layer["qweight"].view(np.uint32)[i, wi]) == word
        wd = [[float(np.float16((int(layer["q"][i, j]) - int(layer["zeros"][j // group, i]))
                                * float(layer["scales"][j // group, i])))
               for j in range(k)] for i in range(n)]
        assert np.array_equal(layer["w_d"], np.array(wd))
        y = o.matmul_ref(x, layer["w_d"], inv)
        for a in range(m):
            for i in range(n):
                acc = 0.0
                for j in range(k):
                    acc += float(x[a, j]) * float(inv[j]) * wd[i][j]
                assert abs(acc - y[a, i]) <= 1e-12 * (1 + abs(acc))


def pin_pack_roundtrip(o, seed=9):
    rng = np.random.default_rng(seed)
    for shape in [(4, 64), (17, 8), (3, 1024)]:
        q = rng.integers(0, 16, size=shape)
        assert np.array_equal(o.unpack_codes(o.pack_codes(q)), q)
        assert np.array_equal(o.unpack_zeros(o.pack_zeros(q)), q)
    # extreme words
    q = np.full((1, 8), 15)
    assert o.pack_codes(q)[0, 0] == -1
    q = np.zeros((1, 8), dtype=int)
    q[0, 7] = 8
    assert o.pack_codes(q)[0, 0] == np.iinfo(np.int32).min


def pin_layout_orientation(o):
    """Scales and zeros are stored [K/G, N]: a layer whose rows differ only in scale
    must show it along the second axis; codes are packed along K."""
    group = 8
    base = np.array([-1.5, -1, -0.5, 0, 4.5, 5, 5.5, 6])   # scale 0.5, zero 3
    w = np.stack([base, base * 2, base * 4])                  # N = 3 rows, K = 8
    q, s, z = o.quantize_rtn(w, group, o.FMT_ASYM)
    assert s.shape == (1, 3) and np.array_equal(s[0], [0.5, 1.0, 2.0])
    assert np.array_equal(z[0], [3, 3, 3])
    w2 = np.concatenate([base, base * 2])[None, :]            # N = 1, K = 16, 2 groups
    q2, s2, z2 = o.quantize_rtn(w2, group, o.FMT_ASYM)
    assert s2.shape == (2, 1) and np.array_equal(s2[:, 0], [0.5, 1.0])


# ------------------------------------------------ objective of the scale search

def _loss_case():
    g = load_golden("awq_loss_hand.txt")
    w = np.zeros((8, 8))
    w[0] = _nums(g["w.row0"])
    x = np.stack([_nums(g["x.row0"]), _nums(g["x.row1"])])
    return g, w, x, int(g["group"])


def pin_loss_hand_value(o):
    """The hand-worked loss of tests/golden/awq_loss_hand.txt: 5 with s = 1 and with
    s = 2 on every channel (asymmetric format)."""
    g, w, x, group = _loss_case()
    for s_val, key in ((1.0, "expect.loss_s1"), (2.0, "expect.loss_s2")):
        loss = o.awq_loss(w, x, np.full(8, s_val), group, o.FMT_ASYM)
        assert loss == float(g[key]), (s_val, loss)


def _grid_layer(rng, n, k, group):
    """W on the 4-bit grid (W = (q - z) s, s of 7 significant bits, codes 0 and 15 in
    every group), so that quantization reproduces it exactly."""
    gs = k // group
    mant = rng.integers(64, 128, size=(gs, n))
    expo = rng.integers(-10, -6, size=(gs, n))
    s = np.ldexp(mant.astype(np.float64), expo)
    z = rng.integers(0, 16, size=(gs, n))
    q = rng.integers(0, 16, size=(n, k))
    q[:, 0::group] = 0
    q[:, 1::group] = 15
    return (q - np.repeat(z.T, group, axis=1)) * np.repeat(s.T, group, axis=1)


def pin_loss_zero_on_grid(o, seed=21, n=8, k=256, group=128):
    """Closed forms of the objective: it is exactly 0 when W is already on the 4-bit
    grid and s = 1, and when W diag(s) is on the grid for a power-of-two s that varies
    from channel to channel (then X diag(s)^-1 and W diag(s) are exact and their
    products equal those of X and W bit for bit). The same W with s = 1 is off the
    grid and gives a positive loss."""
    rng = np.random.default_rng(seed)
    grid = _grid_layer(rng, n, k, group)
    x = rng.standard_normal((4, k))
    assert o.awq_loss(grid, x, np.ones(k), group, o.FMT_ASYM) == 0.0
    s = np.ldexp(1.0, rng.integers(-2, 3, size=k))         # 1/4 .. 4, per channel
    w = grid / s[None, :]                                  # exact: powers of two
    assert np.array_equal(o.fp16_rn(w), w)
    assert o.awq_loss(w, x, s, group, o.FMT_ASYM) == 0.0
    assert o.awq_loss(w, x, np.ones(k), group, o.FMT_ASYM) > 0.0


def pin_scale_search_finds_exact_exponent(o, seed=22, n=8, k=256, group=128):
    """A layer that only the exponent alpha = 1 puts on the grid: W = G diag(m)^-1 with
    G on the grid and channel magnitudes m in {1, 4, 16} that vary within every group,
    calibration rows of magnitude exactly m (so mean |X_cal| = m). alpha = 1 gives
    s = m, the fold gives G back exactly and the loss is 0; alpha = 0, 1/4, 1/2, 3/4
    leave the folded group off the grid, so the search must return alpha = 1."""
    rng = np.random.default_rng(seed)
    grid = _grid_layer(rng, n, k, group)
    m = np.array([1.0, 4.0, 16.0])[rng.integers(0, 3, size=k)]
    w = grid / m[None, :]
    assert np.array_equal(o.fp16_rn(w), w)
    x_cal = m[None, :] * np.where(rng.random((32, k)) < 0.5, -1.0, 1.0)
    best, losses = o.scale_search(w, x_cal, group, o.FMT_ASYM, grid=4)
    assert losses.shape == (5,)
    assert best == 1.0 and losses[4] == 0.0
    assert np.all(losses[:4] > 0.0)


ALL_PINS = [
    pin_fp16_exhaustive, pin_hand_dequant, pin_hand_pack, pin_hand_product,
    pin_hand_requantize, pin_tie_break, pin_on_grid_exact, pin_sym_on_grid,
    pin_degenerate_groups, pin_rtn_error_bound, pin_small_groups, pin_fold_invariance,
    pin_channel_scale, pin_brute_force, pin_pack_roundtrip, pin_layout_orientation,
    pin_loss_hand_value, pin_loss_zero_on_grid, pin_scale_search_finds_exact_exponent,
]


def run_all(o) -> list:
    """Names of the pins that fail for module o."""
    failed = []
    for p in ALL_PINS:
        try:
            p(o)
        except Exception:  # noqa: BLE001  a crash counts as a failed pin
            failed.append(p.__name__)
    return failed


