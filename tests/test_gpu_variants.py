"""Every kernel variant the product entry points can pick, against the CPU oracle.

The dispatcher chooses a decode form (per-group correction or exact dequantization),
a wavefront count (8 or 16), a number of LDS phases for the staged activations, and
for awq_gemm a tiling and a K split, from M, N, K and the workspace. The cases here
are chosen so that each reachable combination runs at least once on a real layer
shape, checked on sampled output rows the oracle computes one by one (within
max|y - y_ref| / max|y_ref| <= 2e-3), and the decode step as the benchmark submits
it (one HIP graph per step, seven launches or four with q|k|v and gate|up fused) is
checked replay after replay.
"""
import numpy as np
import pytest

import oracle
from bit_weight_only_w4a16_amd import synth

torch = pytest.importorskip("torch")
awq = pytest.importorskip("bit_weight_only_w4a16_amd.awq")

pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rel_err(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    return np.max(np.abs(y - y_ref)) / max(np.max(np.abs(y_ref)), 1e-30)


def sampled_rows(n, seed=42, blocks=6):
    rng = np.random.default_rng(seed)
    b = np.unique(np.concatenate([rng.choice(n // 8, blocks, replace=False), [0, n // 8 - 1]]))
    return (b[:, None] * 8 + np.arange(8)[None, :]).ravel()


class Layer:
    """A layer quantized on the GPU, and the oracle's dequantized weights of some rows."""

    def __init__(self, n, k, m, fmt, config=1, layer=0, group=128, rows=None):
        d = synth.layer_inputs(config, m, n, k, layer=layer)
        self.n, self.k, self.m, self.fmt, self.group = n, k, m, fmt, group
        self.x = d["x"]
        w = to_dev(d["w"])
        s_c, self.inv = awq.awq_channel_scale(to_dev(d["x_cal"]), 0.5)
        qw, sc, qz = awq.awq_pack(w, s_c, group, fmt)
        self.packed = awq.awq_repack(qw, sc, qz, n, k, group, fmt)
        del w, qw, sc, qz
        self.rows = sampled_rows(n) if rows is None else rows
        s, inv = oracle.channel_scale(d["x_cal"], 0.5)
        o = oracle.quantize_layer(d["w"][self.rows], s, group, fmt)
        self.w_d, self.inv_ref = o["w_d"], inv

    def y_ref(self, x=None):
        return oracle.matmul_ref(self.x if x is None else x, self.w_d, self.inv_ref)

    def check(self, y, x=None):
        y = y.cpu().numpy()
        assert np.all(np.isfinite(y))
        err = rel_err(y[:, self.rows], self.y_ref(x))
        assert err <= TOL, err
        return err


# ------------------------------------------------ decode: correction form, 16 wavefronts

# (name, N, K, M, fmt, entry). 28672 -> 8192: 512 row tiles of 224 groups: sixteen
# wavefronts, the activations of M = 2 / 3 / 4 rows staged in 2 / 3 / 4 LDS phases;
# 11008 -> 4096: 256 row tiles of 86 groups, sixteen wavefronts, one phase. M = 1 SYM on
# the 70B down layer is the decode launch the benchmark times for that layer.
DECODE_CASES = [
    ("70b_down_sym_m1", 8192, 28672, 1, 1, "gemv"),
    ("70b_down_asym_m2", 8192, 28672, 2, 0, "gemv"),
    ("70b_down_sym_m2", 8192, 28672, 2, 1, "gemv"),
    ("70b_down_asym_m3", 8192, 28672, 3, 0, "gemv"),
    ("70b_down_sym_m3", 8192, 28672, 3, 1, "gemv"),
    ("70b_down_asym_m4", 8192, 28672, 4, 0, "gemv"),
    ("70b_down_sym_m4", 8192, 28672, 4, 1, "gemv"),
    ("7b_down_asym_m2", 4096, 11008, 2, 0, "gemv"),
    ("7b_down_sym_m3", 4096, 11008, 3, 1, "gemv"),
    ("7b_down_asym_m4", 4096, 11008, 4, 0, "gemv"),
    ("7b_down_sym_m4", 4096, 11008, 4, 1, "gemv"),
    # awq_gemm hands M <= 2 to the decode kernel: 2 rows in two LDS phases
    ("70b_down_asym_m2_gemm", 8192, 28672, 2, 0, "gemm"),
    ("70b_down_sym_m2_gemm", 8192, 28672, 2, 1, "gemm"),
    ("70b_up_sym_m1_gemm", 28672, 8192, 1, 1, "gemm"),
]


@pytest.mark.parametrize("name,n,k,m,fmt,fn", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_variants_full_shape(name, n, k, m, fmt, fn):
    L = Layer(n, k, m, fmt, config=4)
    f = awq.awq_gemv if fn == "gemv" else awq.awq_gemm
    ws = awq.workspace(m, n, k, DEV)
    L.check(f(to_dev(L.x), L.inv, L.packed, n, k, 128, fmt, ws=ws))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("m", [2, 3, 4])
def test_decode_correction_form_many_phases(m, fmt):
    """Four row tiles (one workgroup per CU, the 144 KiB LDS budget) of 288 groups:
    the correction form with sixteen wavefronts stages the activations of 2 / 3 / 4
    rows in 2 / 2 / 3 phases, reusing each wavefront's LDS slots from phase to phase."""
    n, k = 64, 36864
    L = Layer(n, k, m, fmt, config=7, rows=np.arange(n))
    L.check(awq.awq_gemv(to_dev(L.x), L.inv, L.packed, n, k, 128, fmt))


# awq_gemv at M > 4 on layers of 512 row tiles or more takes two or four 16-row tiles per
# workgroup (one staging of the activations serves all of them). Ragged cases: 513 and 641
# row tiles (the last tile half full), so the last workgroup's later tiles lie past N.
MULTI_TILE_CASES = [
    # (name, N, K, M, fmt): T = ceil(tiles / 256) up to 768 row tiles, then 2 (4 from M = 12)
    ("t2_ragged_asym_m8", 6152, 1024, 8, 0),     # 385 tiles, 2 per workgroup, last one alone
    ("t2_sym_m5", 8192, 2048, 5, 1),             # 512 tiles, 2 per workgroup
    ("t3_ragged_sym_m12", 10248, 1024, 12, 1),   # 641 tiles, 3 per workgroup
    ("t3_asym_m16_long", 10240, 3072, 16, 0),    # 640 tiles, 3 per workgroup, 24 groups
    ("t3_ragged_asym_m3_corr", 11008, 1024, 3, 0),  # 688 tiles: the correction form, 3 tiles
    ("t3_sym_m2_corr", 12288, 2048, 2, 1),       # 768 tiles: the correction form, 3 tiles
    ("t2_ragged_sym_m4_corr", 12304, 1024, 4, 1),   # 769 tiles: correction form, 2 tiles
    ("t4_ragged_asym_m16", 16400, 1024, 16, 0),  # 1025 tiles, 4 per workgroup
]

@pytest.mark.parametrize("name,n,k,m,fmt", MULTI_TILE_CASES, ids=[c[0] for c in MULTI_TILE_CASES])
def test_gemv_several_tiles_per_workgroup(name, n, k, m, fmt):
    L = Layer(n, k, m, fmt, config=6, rows=np.arange(n))
    y = awq.awq_gemv(to_dev(L.x), L.inv, L.packed, n, k, 128, fmt)
    L.check(y)
    # up to 768 row tiles awq_gemm takes the same kernel on these shapes: the same bits
    if n // 16 <= 768:
        assert awq.awq_workspace_bytes(m, n, k) == 0
        y2 = awq.awq_gemm(to_dev(L.x), L.inv, L.packed, n, k, 128, fmt)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------ wide tiles: banded block order

# M = 1100 gives 9 row blocks of 128: one full band of 8 row blocks and a band of one.
# (name, N, K, M, fmt): 128 x 256 tiles (513 blocks), 128 x 192 tiles (522 blocks), and
# 128 x 192 tiles with K halves inside the workgroup and K split over two workgroups
# (99 blocks).
BAND_CASES = [
    ("band_wn4_asym", 14592, 512, 1100, 0),
    ("band_wn3_sym", 11136, 512, 1100, 1),
    ("band_ks2_sym", 2048, 1024, 1100, 1),
]


@pytest.mark.parametrize("name,n,k,m,fmt", BAND_CASES, ids=[c[0] for c in BAND_CASES])
def test_wide_gemm_partial_band(name, n, k, m, fmt):
    L = Layer(n, k, m, fmt, config=5)
    ws = awq.workspace(m, n, k, DEV)
    L.check(awq.awq_gemm(to_dev(L.x), L.inv, L.packed, n, k, 128, fmt, ws=ws))


# ----------------------------------------------------------- awq_gemm narrow tilings

# M = 48 on a layer of more than 2^26 weights: 64 x 128 workgroup tiles, K split;
# M = 128 on K >= 8192: 128 x 128 tiles with a K split; M = 300 without a workspace on
# N >= 16384: no room for X' or partial sums, so 128 x 128 narrow tiles, unsplit.
NARROW_CASES = [
    ("70b_up_asym_m48", 28672, 8192, 48, 0, True),
    ("70b_up_sym_m48", 28672, 8192, 48, 1, True),
    ("70b_down_asym_m128", 8192, 28672, 128, 0, True),
    ("70b_down_sym_m130", 8192, 28672, 130, 1, True),
    ("8b_gateup_asym_m300_no_ws", 28672, 4096, 300, 0, False),
    ("8b_gateup_sym_m300_no_ws", 28672, 4096, 300, 1, False),
]


@pytest.mark.parametrize("name,n,k,m,fmt,with_ws", NARROW_CASES, ids=[c[0] for c in NARROW_CASES])
def test_gemm_narrow_tilings_full_shape(name, n, k, m, fmt, with_ws):
    L = Layer(n, k, m, fmt, config=4)
    ws = awq.workspace(m, n, k, DEV) if with_ws else None
    L.check(awq.awq_gemm(to_dev(L.x), L.inv, L.packed, n, k, 128, fmt, ws=ws))


def test_gemm_split_k_deterministic_m16():
    """11008 -> 4096 at M = 16: too many groups for the decode kernel's one LDS pass, so
    awq_gemm splits K across workgroups and sums the partials in a second launch, in
    split order: the same bits on every call."""
    n, k, m = 4096, 11008, 16
    assert awq.awq_workspace_bytes(m, n, k) > 0
    L = Layer(n, k, m, 0, config=2)
    ws = awq.workspace(m, n, k, DEV)
    x = to_dev(L.x)
    ys = [awq.awq_gemm(x, L.inv, L.packed, n, k, ws=ws) for _ in range(5)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    L.check(ys[0])


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("group", [32, 64])
def test_small_groups_m3_full_shape(group, fmt):
    """Groups of 32 / 64 at M = 3 on a 7B layer (exact-dequantization decode form)."""
    n, k, m = 11008, 4096, 3
    L = Layer(n, k, m, fmt, config=1, group=group)
    for f in (awq.awq_gemv, awq.awq_gemm):
        L.check(f(to_dev(L.x), L.inv, L.packed, n, k, group, fmt, ws=awq.workspace(m, n, k, DEV, group)))


# --------------------------------------------- the decode step as the benchmark submits it

STEP_7 = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
          ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
STEP_4 = [("qkv", 12288, 4096), ("o", 4096, 4096), ("gate_up", 22016, 4096),
          ("down", 4096, 11008)]


@pytest.mark.parametrize("step", ["7_launches", "4_launches"])
def test_decode_step_graph_replays(step):
    """One HIP graph holding a decoder block's products at M = 1 (seven launches, or four
    with q|k|v as one 4096 -> 12288 layer and gate|up as one 4096 -> 22016 layer),
    replayed several times with eager work and synchronisations in between: every replay
    gives the same bits as the eager calls, and those match the oracle."""
    shapes = STEP_7 if step == "7_launches" else STEP_4
    layers = [Layer(n, k, 1, 0, config=1, layer=20 + j) for j, (_, n, k) in enumerate(shapes)]
    xs = [to_dev(L.x) for L in layers]
    ys = [torch.empty((1, L.n), dtype=torch.float16, device=DEV) for L in layers]

    def run():
        for L, x, y in zip(layers, xs, ys):
            awq.awq_gemv(x, L.inv, L.packed, L.n, L.k, 128, 0, y=y)

    run()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    for L, y in zip(layers, eager):
        L.check(y)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), f"replay {rep}"
        torch.cuda.synchronize()
    del g
