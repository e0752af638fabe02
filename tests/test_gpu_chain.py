"""awq_gemv_chain against the CPU oracle: several M = 1 products in one launch, some
taking an earlier product's output as input.

Two kinds of cases:
  * exact chains: every layer is a signed permutation with entries +-15/16 (asymmetric
    format) or +-7/8 (symmetric), quantized exactly (each group holds one nonzero, whose
    scale 2^-4 / 2^-3 and code the rules reproduce), and the input has a few +-1 entries,
    so every sum the kernel forms is exact in float32 and every output is the binary16
    rounding of the exact product. The chain must then equal the oracle's chain (each
    layer's binary16 output fed to the next) bit for bit: an input read before its
    source layer had finished, or from the previous call, would show;
  * the decoder block of the benchmark on its synthetic data: q, k, v read x; o reads v;
    gate and up read o; down reads up. A layer that reads the caller's x is checked
    within 2e-3 of the oracle; a layer at dependency depth d is checked against the
    oracle's own chain (binary16 outputs fed forward) within 2e-3 (d + 1): its input
    differs from the oracle's by the rounding of each earlier layer (at most about one
    binary16 unit per element, which the product carries into its output as a random
    walk of relative size ~ 2^-11), and the layer adds its own float32 error.
"""
import numpy as np
import pytest

import oracle
from bit_weight_only_w4a16_amd import synth

torch = pytest.importorskip("torch")
awq = pytest.importorskip("bit_weight_only_w4a16_amd.awq")

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def f16(a):
    return oracle.fp16_rn(a)


def rel_err(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    return np.max(np.abs(y - y_ref)) / max(np.max(np.abs(y_ref)), 1e-30)


class ChainLayer:
    """A layer quantized on the GPU and by the oracle from the same fp16 weights."""

    def __init__(self, w, fmt, group=128, s_c=None):
        n, k = w.shape
        self.n, self.k, self.fmt, self.group = n, k, fmt, group
        wd = to_dev(w)
        sc_dev = None if s_c is None else to_dev(s_c)
        qw, sc, qz = awq.awq_pack(wd, sc_dev, group, fmt)
        self.packed = awq.awq_repack(qw, sc, qz, n, k, group, fmt)
        self.w_d = oracle.quantize_layer(w, s_c, group, fmt)["w_d"]

    def spec(self, src=-1, x=None, inv=None):
        d = {"packed": self.packed, "n": self.n, "k": self.k, "group": self.group,
             "fmt": self.fmt, "src": src}
        if x is not None:
            d["x"] = to_dev(x)
        if inv is not None:
            d["inv_s_c"] = to_dev(inv)
        return d


def oracle_chain(layers, srcs, x, invs=None):
    """The oracle's outputs of a chain: layer i reads x (src -1) or the binary16 output
    of layer srcs[i]."""
    outs = []
    for i, (L, s) in enumerate(zip(layers, srcs)):
        inp = x if s < 0 else outs[s]
        inv = None if invs is None else invs[i]
        outs.append(f16(oracle.matmul_ref(inp, L.w_d, inv)))
    return outs


# ------------------------------------------------------------------- exact chains

# layers, their sources; N = K = 2048 (16 groups of 128, 128 row tiles per layer).
# A 4-deep dependent chain with an independent layer and a second reader of layer 1.
EXACT_SRCS = [-1, 0, 1, -1, 2, 1]


def exact_chain(fmt, seed):
    n = 2048
    value = 15.0 / 16.0 if fmt == awq.FMT_ASYM else 7.0 / 8.0
    return [ChainLayer(synth.signed_permutation(n, seed + 17 * i, value), fmt)
            for i in range(len(EXACT_SRCS))]


def nonzeros_per_group(v, group=128):
    return int(np.max(np.count_nonzero(np.asarray(v).reshape(-1, group), axis=1)))


@pytest.mark.parametrize("fmt", [awq.FMT_ASYM, awq.FMT_SYM8])
def test_chain_exact_bit_for_bit(fmt):
    layers = exact_chain(fmt, seed=900 + fmt)
    state = awq.chain_state(DEV)
    # two calls in a row with different inputs: the second must not see the first's outputs
    for call, xseed in enumerate((11, 12)):
        x = synth.sparse_signs(2048, 8, seed=xseed + 10 * fmt)
        # power-of-two channel scales on two of the layers (exact products)
        rng = np.random.default_rng(70 + call)
        inv0 = np.exp2(rng.integers(-1, 2, 2048)).astype(np.float16)
        inv2 = np.exp2(rng.integers(-1, 2, 2048)).astype(np.float16)
        invs = [inv0, None, inv2, None, None, None]
        refs = oracle_chain(layers, EXACT_SRCS, x.astype(np.float64), invs)
        # the exactness argument needs at most 4 nonzero inputs per 128-channel group
        assert nonzeros_per_group(x) <= 4
        assert all(nonzeros_per_group(r) <= 4 for r in refs)
        specs = [L.spec(s, x if s < 0 else None, inv)
                 for L, s, inv in zip(layers, EXACT_SRCS, invs)]
        outs = awq.awq_gemv_chain(specs, state)
        torch.cuda.synchronize()
        assert awq.chain_errors(state) == 0
        for i, (y, r) in enumerate(zip(outs, refs)):
            yb = y.cpu().numpy().astype(np.float64)
            assert np.array_equal(yb, r), (call, i, np.max(np.abs(yb - r)))
            assert np.count_nonzero(r) > 0


def test_chain_exact_single_layer_and_fan_out():
    """One layer alone, and three layers that all read the same source."""
    n = 2048
    ls = [ChainLayer(synth.signed_permutation(n, 300 + i, 15.0 / 16.0), awq.FMT_ASYM)
          for i in range(4)]
    state = awq.chain_state(DEV)
    x = synth.sparse_signs(n, 6, seed=5)
    for srcs in ([-1], [-1, 0, 0, 0]):
        use = ls[:len(srcs)]
        refs = oracle_chain(use, srcs, x.astype(np.float64))
        outs = awq.awq_gemv_chain([L.spec(s, x if s < 0 else None) for L, s in zip(use, srcs)], state)
        torch.cuda.synchronize()
        assert awq.chain_errors(state) == 0
        for y, r in zip(outs, refs):
            assert np.array_equal(y.cpu().numpy().astype(np.float64), r)


# ------------------------------------------------------------ the decoder block

# (name, N, K, src): the benchmark's 7B decoder block at M = 1
BLOCK = [("q", 4096, 4096, -1), ("k", 4096, 4096, -1), ("v", 4096, 4096, -1),
         ("o", 4096, 4096, 2), ("gate", 11008, 4096, 3), ("up", 11008, 4096, 3),
         ("down", 4096, 11008, 5)]


def depth_of(srcs):
    d = []
    for s in srcs:
        d.append(0 if s < 0 else d[s] + 1)
    return d


@pytest.fixture(scope="module")
def block():
    """The block's layers quantized on the GPU (channel scale, fold, pack, repack) and by
    the oracle from the same seeded weights and calibration rows, the input x, and the
    oracle's chain of outputs."""
    layers, invs, invs_ref = [], [], []
    for j, (name, n, k, src) in enumerate(BLOCK):
        d = synth.layer_inputs(1, 1, n, k, layer=j)
        s_dev, inv_dev = awq.awq_channel_scale(to_dev(d["x_cal"]), 0.5)
        s_ref, inv_ref = oracle.channel_scale(d["x_cal"], 0.5)
        L = ChainLayer.__new__(ChainLayer)
        L.n, L.k, L.fmt, L.group = n, k, awq.FMT_ASYM, 128
        qw, sc, qz = awq.awq_pack(to_dev(d["w"]), s_dev, 128, awq.FMT_ASYM)
        L.packed = awq.awq_repack(qw, sc, qz, n, k, 128, awq.FMT_ASYM)
        L.w_d = oracle.quantize_layer(d["w"], s_ref, 128, awq.FMT_ASYM)["w_d"]
        layers.append(L)
        invs.append(inv_dev)
        invs_ref.append(inv_ref)
    x = synth.layer_inputs(1, 1, 4096, 4096, layer=0)["x"]
    srcs = [b[3] for b in BLOCK]
    refs = oracle_chain(layers, srcs, x.astype(np.float64), invs_ref)
    return layers, invs, x, srcs, refs


def block_specs(block, ys=None):
    layers, invs, x, srcs, _ = block
    xd = to_dev(x)
    specs = []
    for i, (L, s, inv) in enumerate(zip(layers, srcs, invs)):
        sp = {"packed": L.packed, "n": L.n, "k": L.k, "src": s, "inv_s_c": inv}
        if s < 0:
            sp["x"] = xd
        if ys is not None:
            sp["y"] = ys[i]
        specs.append(sp)
    return specs


def run_block(block, state, ys=None):
    return awq.awq_gemv_chain(block_specs(block, ys), state)


def test_chain_decoder_block_against_oracle(block):
    layers, invs, x, srcs, refs = block
    state = awq.chain_state(DEV)
    outs = run_block(block, state)
    torch.cuda.synchronize()
    assert awq.chain_errors(state) == 0
    for (name, n, k, s), d, y, r in zip(BLOCK, depth_of(srcs), outs, refs):
        yy = y.cpu().numpy()
        assert np.all(np.isfinite(yy)), name
        err = rel_err(yy, r)
        print(f"chain {name}: depth {d}, max|y - y_ref| / max|y_ref| = {err:.2e}")
        assert err <= TOL * (d + 1), (name, d, err)


def test_chain_decoder_block_matches_separate_products(block):
    """Each layer of the chain agrees with awq_gemv run separately on the chain's own
    input, within 2e-3 (the same per-group arithmetic; the two split K over different
    numbers of wavefronts, so the float32 sums are added in another order)."""
    layers, invs, x, srcs, _ = block
    state = awq.chain_state(DEV)
    outs = run_block(block, state)
    for (name, n, k, s), L, inv, y in zip(BLOCK, layers, invs, outs):
        inp = to_dev(x) if s < 0 else outs[s]
        ref = awq.awq_gemv(inp, inv, L.packed, n, k, 128, awq.FMT_ASYM)
        err = rel_err(y.cpu().numpy(), ref.cpu().numpy().astype(np.float64))
        assert err <= TOL, (name, err)
    torch.cuda.synchronize()
    assert awq.chain_errors(state) == 0


def test_chain_repeatable_and_graph_replays(block):
    """Repeated calls give the same bits; the chain captured in a HIP graph replays with
    the same bits, with eager work and synchronisation between replays (the state
    buffer is left as found by every call)."""
    state = awq.chain_state(DEV)
    first = [y.clone() for y in run_block(block, state)]
    again = run_block(block, state)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b)
    ys = [torch.empty_like(y) for y in first]
    specs = block_specs(block, ys)  # device tensors prepared before the capture
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        awq.awq_gemv_chain(specs, state)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        awq.awq_gemv_chain(specs, state)
    for rep in range(4):
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(first, ys):
            assert torch.equal(a, b), rep
        scratch = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        assert torch.isfinite(scratch)
    assert awq.chain_errors(state) == 0
    # every call leaves the done counter (word 32) and the layer counters (from word 64) at zero
    assert int(state[128:].view(torch.int32).abs().sum().item()) == 0
