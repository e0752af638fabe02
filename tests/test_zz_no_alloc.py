"""awq_gemm_noalloc (the library's own device scratch) against awq_gemm with a caller
workspace: the same kernels and split choices, so the same bits, on two calls in a row,
the second with a smaller input; and both within 2e-3 of the CPU oracle."""
import numpy as np
import pytest

import oracle
from bit_weight_only_w4a16_amd import synth

torch = pytest.importorskip("torch")
awq = pytest.importorskip("bit_weight_only_w4a16_amd.awq")

pytestmark = pytest.mark.gpu

DEV = "cuda"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def case(n, k, m, fmt, seed):
    d = synth.layer_inputs(seed, m, n, k)
    s_c, inv = awq.awq_channel_scale(to_dev(d["x_cal"]), 0.5)
    qw, sc, qz = awq.awq_pack(to_dev(d["w"]), s_c, 128, fmt)
    packed = awq.awq_repack(qw, sc, qz, n, k, 128, fmt)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), np.arange(n // 2, n // 2 + 8)]))
    s, inv_ref = oracle.channel_scale(d["x_cal"], 0.5)
    w_d = oracle.quantize_layer(d["w"][rows], s, 128, fmt)["w_d"]
    y_ref = oracle.matmul_ref(d["x"], w_d, inv_ref)
    return to_dev(d["x"]), inv, packed, rows, y_ref


@pytest.mark.parametrize("fmt", [0, 1])
def test_noalloc_matches_gemm_on_two_calls(fmt):
    # 1) M = 300 on 4096 -> 512: X' formed into the scratch and K split across workgroups
    #    (partial sums after X'); 2) a smaller call, M = 16 on 11008 -> 4096: narrow tiles
    #    with K split (partial sums at the start of the scratch, over the first call's X')
    for n, k, m, seed in ((512, 4096, 300, 31), (4096, 11008, 16, 32)):
        need = awq.awq_workspace_bytes(m, n, k)
        assert 0 < need <= 64 << 20
        x, inv, packed, rows, y_ref = case(n, k, m, fmt, seed)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        y_ws = awq.awq_gemm(x, inv, packed, n, k, 128, fmt, ws=ws)
        y_na = torch.empty((m, n), dtype=torch.float16, device=DEV)
        awq.awq_gemm_noalloc(x, inv, packed, n, k, 128, fmt, y=y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))
        y = y_na.cpu().numpy().astype(np.float64)[:, rows]
        assert np.max(np.abs(y - y_ref)) / np.max(np.abs(y_ref)) <= 2e-3


def test_noalloc_needs_no_workspace_path_and_rejects_oversize():
    """M = 1 needs no workspace (the scratch is not touched); a call needing more than
    64 MiB is refused before any launch."""
    n, k = 4096, 4096
    x, inv, packed, rows, y_ref = case(n, k, 1, 0, 33)
    y_na = awq.awq_gemm_noalloc(x, inv, packed, n, k)
    y_ws = awq.awq_gemm(x, inv, packed, n, k)
    torch.cuda.synchronize()
    assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))
    big_m, big_k = 4096, 28672
    assert awq.awq_workspace_bytes(big_m, 8192, big_k) > 64 << 20
    xs = torch.zeros((big_m, big_k), dtype=torch.float16, device=DEV)
    with pytest.raises(awq.AwqError) as e:
        awq.awq_gemm_noalloc(xs, None, torch.zeros(awq.awq_repacked_bytes(8192, big_k), dtype=torch.uint8,
                                                   device=DEV), 8192, big_k)
    assert e.value.code == 4
