"""The C-ABI library without a GPU: it loads, exports every declared entry point, and
rejects bad arguments with the documented status before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

awq = pytest.importorskip("bit_weight_only_w4a16_amd.awq")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(awq.LIB_PATH):
        pytest.skip("library not built")
    return awq.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(awq.EXPORTS) == names


def test_probe_library_exports_its_header():
    """The benchmark's ceiling probes live in their own library with their own header."""
    from bit_weight_only_w4a16_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        pytest.skip("probe library not built")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "awq_probe.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)))
    assert names == ["awq_probe_empty", "awq_probe_mfma_alu", "awq_probe_shapes",
                     "awq_probe_stream_read"]
    probe = ctypes.CDLL(B.PROBE_LIB)
    for n in names:
        assert hasattr(probe, n), n
    assert probe.awq_probe_shapes() == 4
    probe.awq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
    assert probe.awq_probe_stream_read(None, 1024, 0, None, None) == 1   # checked before launch
    assert probe.awq_probe_stream_read(16, 1 << 31, 0, 16, None) == 1
    assert probe.awq_probe_stream_read(8, 1024, 0, 16, None) == 3
    probe.awq_probe_mfma_alu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    assert probe.awq_probe_mfma_alu(None, 0, 256, 10, None) == 1
    assert probe.awq_probe_mfma_alu(16, 5, 256, 10, None) == 1
    assert probe.awq_probe_mfma_alu(16, 0, 0, 10, None) == 1
    assert probe.awq_probe_mfma_alu(16, 0, 4097, 10, None) == 1


def test_gemm_noalloc_checks_before_any_launch(lib):
    """awq_gemm_noalloc runs awq_gemm's argument checks and refuses a product whose
    workspace would exceed its 64 MiB device scratch, all before touching the GPU."""
    f = lib.awq_gemm_noalloc
    a = 1 << 20   # 16-byte aligned stand-in addresses (never dereferenced)
    assert f(None, None, a, 4, 4096, 4096, 128, 0, a, None) == INVALID
    assert f(a, None, a, 4, 4096, 4097, 128, 0, a, None) == INVALID
    assert f(a + 8, None, a, 4, 4096, 4096, 128, 0, a, None) == MISALIGNED
    assert f(a, None, a, 4, 4096, 4096, 16, 0, a, None) == UNSUPPORTED
    assert awq.awq_workspace_bytes(4096, 8192, 28672) > 64 << 20
    assert f(a, None, a, 4096, 8192, 28672, 128, 0, a, None) == WORKSPACE
    assert f(a, None, a, 0, 4096, 4096, 128, 0, a, None) == OK   # M = 0: no launch


def test_chain_checks_before_any_launch(lib):
    """awq_gemv_chain validates every layer descriptor before launching anything."""
    f = lib.awq_gemv_chain
    a = 1 << 20   # 16-byte aligned stand-in addresses (never dereferenced)
    state = 1 << 24

    def layers(*specs):
        arr = (awq.ChainLayer * max(1, len(specs)))()
        for i, sp in enumerate(specs):
            d = dict(x=a, inv_s_c=None, packed=a, y=a + 4096 * (i + 1), N=4096, K=4096,
                     group=128, fmt=0, src=-1, reserved=0)
            d.update(sp)
            arr[i] = awq.ChainLayer(**d)
        return ctypes.cast(arr, ctypes.c_void_p)

    ok = layers({}, {"src": 0, "x": None})
    assert f(ok, 0, state, None) == OK                     # no layers: nothing to launch
    assert f(None, 1, state, None) == INVALID
    assert f(ok, 2, None, None) == INVALID
    assert f(ok, -1, state, None) == INVALID
    assert f(layers(*[{}] * 9), 9, state, None) == UNSUPPORTED   # more than 8 layers
    assert f(layers({"x": None}), 1, state, None) == INVALID        # src -1 needs x
    assert f(layers({"packed": None}), 1, state, None) == INVALID
    assert f(layers({"y": None}), 1, state, None) == INVALID
    assert f(layers({}, {"src": 1}), 2, state, None) == INVALID    # src must be earlier
    assert f(layers({}, {"src": -2}), 2, state, None) == INVALID
    assert f(layers({"N": 11008}, {"src": 0, "K": 4096}), 2, state, None) == INVALID  # N != K
    assert f(layers({"N": 4100}), 1, state, None) == INVALID       # N % 8
    assert f(layers({"group": 64}), 1, state, None) == UNSUPPORTED  # groups of 128 and up
    assert f(layers({"K": 512, "x": a}), 1, state, None) == UNSUPPORTED   # K < 1024
    assert f(layers({"K": 28672}), 1, state, None) == UNSUPPORTED  # K > 16384
    assert f(layers({"x": a + 8}), 1, state, None) == MISALIGNED
    assert f(layers({"inv_s_c": a + 2}), 1, state, None) == MISALIGNED
    assert f(ok, 2, state + 4, None) == MISALIGNED
    assert awq.awq_chain_state_bytes() > 0 and awq.awq_chain_state_bytes() % 256 == 0


def test_status_strings(lib):
    for code in range(6):
        s = awq.status_string(code)
        assert isinstance(s, str) and s
    assert awq.status_string(99) == "unknown status"
    assert awq.awq_layout_version() == 3


def test_sizes():
    # codes N*K/2 + scales 2*N*K/128 + zeros N*K/256, regions 256-byte aligned
    assert awq.awq_repacked_bytes(4096, 4096) == 8388608 + 262144 + 65536
    assert awq.awq_repacked_bytes(4096, 4096, 128, awq.FMT_SYM8) == 8388608 + 262144
    assert awq.awq_repacked_bytes(100, 256) == 0          # N % 8 != 0
    assert awq.awq_repacked_bytes(64, 200) == 0           # K % 128 != 0
    assert awq.awq_repacked_bytes(64, 384, 96) == 0       # unsupported group
    assert awq.awq_repacked_bytes(64, 200, 8) == 0        # K not a multiple of 128
    # groups of 64 / 32: two / four scale sets per 1 KiB unit; >= 128: one set per unit
    # (4 tiles x 2 units: codes 8192 B; scales 4 x 2 x S x 32 B; zeros 4 x 2 x S x 8 B;
    # regions 256-byte aligned)
    assert awq.awq_repacked_bytes(64, 256, 64) == 8192 + 512 + 256
    assert awq.awq_repacked_bytes(64, 256, 32) == 8192 + 1024 + 256
    assert awq.awq_repacked_bytes(64, 256, 256) == awq.awq_repacked_bytes(64, 256, 128)
    assert awq.awq_workspace_bytes(0, 4096, 4096) == 0
    # partial sums in the workspace only where few output blocks need K split across
    # workgroups (4096 output columns at M = 16: 64 blocks, four workgroups per block);
    # with many blocks (11008 columns) K is split inside the workgroup, no workspace
    assert awq.awq_workspace_bytes(16, 4096, 11008) == 4 * 16 * 4096 * 4
    assert awq.awq_workspace_bytes(16, 11008, 4096) == 0
    # up to 16 rows on at most 256 row tiles the decode kernel runs: no workspace
    assert awq.awq_workspace_bytes(16, 4096, 4096) == 0
    assert awq.awq_workspace_bytes(8, 4096, 11008) == 0
    assert awq.awq_workspace_bytes(12, 4096, 11008) > 0
    # large M: X' = X * inv_s_c formed once, M x K binary16
    assert awq.awq_workspace_bytes(2048, 4096, 4096) == 2048 * 4096 * 2
    # M >= 256 with few output blocks: X' (256-byte aligned) then float32 sums of the
    # K splits (2 x 32 blocks of 128 x 256: 256 / 64 = 4 splits; 2 x 112 blocks: none)
    assert awq.awq_workspace_bytes(256, 8192, 28672) == 256 * 28672 * 2 + 4 * 256 * 8192 * 4
    assert awq.awq_workspace_bytes(256, 28672, 8192) == 256 * 8192 * 2


def test_padded_layout_size():
    # 72 rows -> 5 tiles of 16; K = 256 -> 2 groups of 128
    codes = 5 * 2 * 1024
    scales = 5 * 2 * 16 * 2
    zeros_off = (codes + scales + 255) // 256 * 256
    total = (zeros_off + 5 * 2 * 8 + 255) // 256 * 256
    assert awq.awq_repacked_bytes(72, 256) == total
    assert awq.awq_repacked_bytes(72, 256, 128, awq.FMT_SYM8) == (codes + scales + 255) // 256 * 256


P = 4096  # an aligned stand-in address; never dereferenced because validation fails


@pytest.mark.parametrize("args,code", [
    ((None, None, P, 1, 64, 128, 128, 0, P, None, 0, None), INVALID),      # x NULL
    ((P, None, None, 1, 64, 128, 128, 0, P, None, 0, None), INVALID),      # packed NULL
    ((P, None, P, 1, 64, 128, 128, 0, None, None, 0, None), INVALID),      # y NULL
    ((P, None, P, 1, 60, 128, 128, 0, P, None, 0, None), INVALID),         # N % 8
    ((P, None, P, 1, 64, 100, 128, 0, P, None, 0, None), INVALID),         # K % group
    ((P, None, P, 1, 64, 128, 128, 2, P, None, 0, None), INVALID),         # fmt
    ((P, None, P, -1, 64, 128, 128, 0, P, None, 0, None), INVALID),        # M < 0
    ((P, None, P, 1, 64, 384, 96, 0, P, None, 0, None), UNSUPPORTED),      # group 96
    ((P + 2, None, P, 1, 64, 128, 128, 0, P, None, 0, None), MISALIGNED),  # x
    ((P, P + 8, P, 1, 64, 128, 128, 0, P, None, 0, None), MISALIGNED),     # inv_s_c
    ((P, None, P, 1, 64, 128, 128, 0, P, None, 16, None), INVALID),        # ws NULL, bytes
    ((P, None, P, 17, 64, 128, 128, 0, P, None, 0, None), UNSUPPORTED),    # M > 16 (gemv)
    ((None, None, None, 0, 64, 128, 128, 0, None, None, 0, None), OK),     # M == 0: no-op
])
def test_gemv_validation(lib, args, code):
    assert lib.awq_gemv(*args) == code


def test_gemm_validation(lib):
    assert lib.awq_gemm(None, None, None, 0, 64, 128, 128, 0, None, None, 0, None) == OK
    assert lib.awq_gemm(P, None, P, 9, 64, 100, 128, 0, P, None, 0, None) == INVALID
    assert lib.awq_gemm(P, None, P, 9, 64, 384, 96, 0, P, None, 0, None) == UNSUPPORTED
    assert lib.awq_gemm(P, None, P + 4, 9, 64, 128, 128, 0, P, None, 0, None) == MISALIGNED


def test_layer_size_limit(lib):
    # N * K must stay below 2^31 (offsets into one layer fit in 31 bits)
    k = 1 << 16
    n_ok, n_big = (1 << 15) - 8, 1 << 15
    assert lib.awq_repacked_bytes(n_ok, k, 128, 0) > 0
    assert lib.awq_repacked_bytes(n_big, k, 128, 0) == 0
    assert lib.awq_gemv(P, None, P, 1, n_big, k, 128, 0, P, None, 0, None) == UNSUPPORTED
    assert lib.awq_gemm(P, None, P, 16, n_big, k, 128, 0, P, None, 0, None) == UNSUPPORTED


def test_pack_and_repack_validation(lib):
    # qzeros must be given for the asymmetric format and NULL for the symmetric one
    assert lib.awq_pack(P, None, 64, 128, 128, 0, P, P, None, None) == INVALID
    assert lib.awq_pack(P, None, 64, 128, 128, 1, P, P, P, None) == INVALID
    assert lib.awq_pack(None, None, 64, 128, 128, 0, P, P, P, None) == INVALID
    assert lib.awq_pack(P, P + 2, 64, 128, 128, 0, P, P, P, None) == MISALIGNED
    assert lib.awq_repack(P, P, P, 64, 128, 128, 0, P, 16, None) == WORKSPACE
    assert lib.awq_repack(P, P, None, 64, 128, 128, 0, P, 1 << 20, None) == INVALID
    assert lib.awq_dequant(P, P, P, 1, 64, 128, 128, 0, P, None) == INVALID   # gfx950 + scales
    assert lib.awq_dequant(P, None, None, 7, 64, 128, 128, 1, P, None) == INVALID
    assert lib.awq_dequant(P, None, None, 0, 64, 128, 128, 1, P, None) == INVALID  # no scales


def test_channel_scale_validation(lib):
    assert lib.awq_channel_scale(None, 32, 512, 0.5, P, None, None) == INVALID
    assert lib.awq_channel_scale(P, 0, 512, 0.5, P, None, None) == INVALID
    assert lib.awq_channel_scale(P, 9000, 512, 0.5, P, None, None) == INVALID
    assert lib.awq_channel_scale(P, 32, 512, 1.5, P, None, None) == INVALID
    assert lib.awq_channel_scale(P, 32, 512, float("nan"), P, None, None) == INVALID
    assert lib.awq_channel_scale(P, 32, 512, 0.5, P + 2, None, None) == MISALIGNED


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        awq.awq_gemv(torch.zeros(1, 128, dtype=torch.float16), None,
                     torch.zeros(16, dtype=torch.uint8), 64, 128)


def test_ctypes_signature_matches_header():
    text = open(HEADER).read()
    for name, (_res, argtypes) in awq._SIGNATURES.items():
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text, flags=re.S)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(argtypes), name
    _ = ctypes


def test_scale_search_validation(lib):
    need = lib.awq_scale_search_workspace_bytes(32, 256, 1024, 128, 0)
    assert need > 256 * 1024 // 2                                   # holds a quantized layer
    assert lib.awq_scale_search_workspace_bytes(0, 256, 1024, 128, 0) == 0
    assert lib.awq_scale_search_workspace_bytes(257, 256, 1024, 128, 0) == 0
    args = [P, P, 32, 256, 1024, 128, 0, 20, P, P, P, need, None]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.awq_scale_search(*a)
    assert call(a0=None) == INVALID                   # w NULL
    assert call(a2=0) == INVALID                      # rows
    assert call(a2=257) == INVALID
    assert call(a7=0) == INVALID                      # grid
    assert call(a5=16) == UNSUPPORTED                 # group 16
    assert call(a8=P + 4) == MISALIGNED               # losses
    assert call(a1=P + 2) == MISALIGNED               # x_cal
    assert call(a11=need - 1) == WORKSPACE
