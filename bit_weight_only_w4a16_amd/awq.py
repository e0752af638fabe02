"""Thin ctypes binding of the gfx950 C-ABI library ``libawq_gfx950.so``.

Every function here has the name of the C entry point it calls and only marshals
arguments: it checks device, dtype and contiguity, allocates outputs with PyTorch
(device memory is PyTorch's, streams are PyTorch's current stream) and raises
``AwqError`` on a non-zero status. All arithmetic happens in the library's HIP
kernels; there is no fallback. If the library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

FMT_ASYM = 0
FMT_SYM8 = 1
LAYOUT_CANONICAL = 0
LAYOUT_GFX950 = 1
GROUP = 128

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libawq_gfx950.so")

_lib = None
_lib_lock = threading.Lock()

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

_SIGNATURES = {
    "awq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "awq_layout_version": (ctypes.c_int, []),
    "awq_channel_scale": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_double, _vp, _vp, _vp]),
    "awq_pack": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "awq_repacked_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "awq_repack": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _sz, _vp]),
    "awq_dequant": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp]),
    "awq_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "awq_gemv": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _sz, _vp]),
    "awq_gemm": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _sz, _vp]),
    "awq_gemm_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp]),
    "awq_scale_search_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "awq_scale_search": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _vp,
                                        _vp, _sz, _vp]),
    "awq_chain_state_bytes": (_sz, []),
    "awq_gemv_chain": (ctypes.c_int, [_vp, _i32, _vp, _vp]),
}
EXPORTS = tuple(_SIGNATURES)


class ChainLayer(ctypes.Structure):
    """awq_chain_layer of awq.h."""
    _fields_ = [("x", _vp), ("inv_s_c", _vp), ("packed", _vp), ("y", _vp), ("N", _i64),
                ("K", _i64), ("group", _i32), ("fmt", _i32), ("src", _i32), ("reserved", _i32)]


CHAIN_MAX_LAYERS = 8


class AwqError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} (status {code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load the library once (after PyTorch, so both share PyTorch's HIP runtime)."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is not built; run `python -m bit_weight_only_w4a16_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def status_string(code: int) -> str:
    return lib().awq_status_string(int(code)).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise AwqError(rc, what)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, name, dtype) -> int | None:
    return None if t is None else _dev(t, name, dtype)


def _shape(t, name, shape) -> None:
    """The library sees raw pointers: every buffer's extent is checked here."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _at_least(t, name, nbytes: int) -> None:
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _same_device(ref: torch.Tensor, **named) -> None:
    for name, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# ------------------------------------------------------------------- entry points

def awq_layout_version() -> int:
    return lib().awq_layout_version()


def awq_channel_scale(x_cal: torch.Tensor, alpha: float = 0.5, want_inv: bool = True):
    """(s_c, inv_s_c) fp16 [K] from calibration rows x_cal fp16 [rows, K]."""
    if x_cal.dim() != 2:
        raise ValueError("x_cal must be [rows, K]")
    rows, k = x_cal.shape
    s_c = torch.empty(k, dtype=torch.float16, device=x_cal.device)
    inv = torch.empty_like(s_c) if want_inv else None
    _check(lib().awq_channel_scale(_dev(x_cal, "x_cal", torch.float16), rows, k, float(alpha),
                                   s_c.data_ptr(), _opt(inv, "inv_s_c", torch.float16),
                                   _stream(x_cal.device)), "awq_channel_scale")
    return s_c, inv


def awq_pack(w: torch.Tensor, s_c: torch.Tensor | None = None, group: int = GROUP,
             fmt: int = FMT_ASYM):
    """Fold s_c into W fp16 [N, K], quantize and pack: (qweight, scales, qzeros|None)."""
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    dev = w.device
    _shape(s_c, "s_c", (k,))
    _same_device(w, s_c=s_c)
    if group <= 0 or k % group != 0:
        raise ValueError("group must divide K")
    qweight = torch.empty((n, k // 8), dtype=torch.int32, device=dev)
    scales = torch.empty((k // group, n), dtype=torch.float16, device=dev)
    qzeros = torch.empty((k // group, n // 8), dtype=torch.int32, device=dev) if fmt == FMT_ASYM else None
    _check(lib().awq_pack(_dev(w, "w", torch.float16), _opt(s_c, "s_c", torch.float16), n, k,
                          group, fmt, qweight.data_ptr(), scales.data_ptr(),
                          _opt(qzeros, "qzeros", torch.int32), _stream(dev)), "awq_pack")
    return qweight, scales, qzeros


def awq_repacked_bytes(n: int, k: int, group: int = GROUP, fmt: int = FMT_ASYM) -> int:
    return int(lib().awq_repacked_bytes(n, k, group, fmt))


def awq_repack(qweight, scales, qzeros, n: int, k: int, group: int = GROUP,
               fmt: int = FMT_ASYM) -> torch.Tensor:
    """Canonical packed tensors -> gfx950 packed buffer (uint8)."""
    nbytes = awq_repacked_bytes(n, k, group, fmt)
    if nbytes == 0:
        raise ValueError("invalid layer shape")
    _shape(qweight, "qweight", (n, k // 8))
    _shape(scales, "scales", (k // group, n))
    _shape(qzeros, "qzeros", (k // group, n // 8))
    _same_device(qweight, scales=scales, qzeros=qzeros)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=qweight.device)
    _check(lib().awq_repack(_dev(qweight, "qweight", torch.int32),
                            _dev(scales, "scales", torch.float16),
                            _opt(qzeros, "qzeros", torch.int32), n, k, group, fmt,
                            packed.data_ptr(), nbytes, _stream(qweight.device)), "awq_repack")
    return packed


def awq_dequant(w, scales, qzeros, layout: int, n: int, k: int, group: int = GROUP,
                fmt: int = FMT_ASYM, out: torch.Tensor | None = None) -> torch.Tensor:
    """W_d fp16 [N, K] from the canonical (layout 0) or gfx950 (layout 1) format."""
    if out is None:
        out = torch.empty((n, k), dtype=torch.float16, device=w.device)
    _shape(out, "out", (n, k))
    wdt = torch.int32 if layout == LAYOUT_CANONICAL else torch.uint8
    if layout == LAYOUT_CANONICAL and k % 8 == 0 and group > 0 and k % group == 0:
        _shape(w, "w", (n, k // 8))
        _shape(scales, "scales", (k // group, n))
        _shape(qzeros, "qzeros", (k // group, n // 8))
    elif layout == LAYOUT_GFX950:
        _at_least(w, "packed", awq_repacked_bytes(n, k, group, fmt))
    _same_device(w, scales=scales, qzeros=qzeros, out=out)
    _check(lib().awq_dequant(_dev(w, "w", wdt), _opt(scales, "scales", torch.float16),
                             _opt(qzeros, "qzeros", torch.int32), layout, n, k, group, fmt,
                             _dev(out, "out", torch.float16), _stream(w.device)), "awq_dequant")
    return out


def awq_workspace_bytes(m: int, n: int, k: int, group: int = GROUP) -> int:
    return int(lib().awq_workspace_bytes(m, n, k, group))


def _product(fn_name, x, inv_s_c, packed, n, k, group, fmt, y, ws):
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x must have K columns")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    _shape(y, "y", (m, n))
    _shape(inv_s_c, "inv_s_c", (k,))
    _at_least(packed, "packed", awq_repacked_bytes(n, k, group, fmt))
    _same_device(x, inv_s_c=inv_s_c, packed=packed, y=y, ws=ws)
    ws_ptr, ws_bytes = (None, 0) if ws is None else (_dev(ws, "ws", torch.uint8), ws.numel())
    rc = getattr(lib(), fn_name)(_dev(x, "x", torch.float16), _opt(inv_s_c, "inv_s_c", torch.float16),
                                 _dev(packed, "packed", torch.uint8), m, n, k, group, fmt,
                                 _dev(y, "y", torch.float16), ws_ptr, ws_bytes, _stream(x.device))
    _check(rc, fn_name)
    return y


def awq_gemv(x, inv_s_c, packed, n: int, k: int, group: int = GROUP, fmt: int = FMT_ASYM,
             y=None, ws=None) -> torch.Tensor:
    """Decode product, 1 <= M <= 16."""
    return _product("awq_gemv", x, inv_s_c, packed, n, k, group, fmt, y, ws)


def awq_gemm(x, inv_s_c, packed, n: int, k: int, group: int = GROUP, fmt: int = FMT_ASYM,
             y=None, ws=None) -> torch.Tensor:
    """Matrix-core product, any M >= 1."""
    return _product("awq_gemm", x, inv_s_c, packed, n, k, group, fmt, y, ws)


def awq_gemm_noalloc(x, inv_s_c, packed, n: int, k: int, group: int = GROUP,
                     fmt: int = FMT_ASYM, y=None) -> torch.Tensor:
    """awq_gemm with the library's own device scratch instead of a caller workspace (the
    call allocates nothing; pass `y` to allocate nothing on this side either)."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x must have K columns")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    _shape(y, "y", (m, n))
    _shape(inv_s_c, "inv_s_c", (k,))
    _at_least(packed, "packed", awq_repacked_bytes(n, k, group, fmt))
    _same_device(x, inv_s_c=inv_s_c, packed=packed, y=y)
    _check(lib().awq_gemm_noalloc(_dev(x, "x", torch.float16), _opt(inv_s_c, "inv_s_c", torch.float16),
                                  _dev(packed, "packed", torch.uint8), m, n, k, group, fmt,
                                  _dev(y, "y", torch.float16), _stream(x.device)), "awq_gemm_noalloc")
    return y


def awq_scale_search_workspace_bytes(rows: int, n: int, k: int, group: int = GROUP,
                                     fmt: int = FMT_ASYM) -> int:
    return int(lib().awq_scale_search_workspace_bytes(rows, n, k, group, fmt))


def awq_scale_search(w, x_cal, group: int = GROUP, fmt: int = FMT_ASYM, grid: int = 20,
                     ws=None):
    """AWQ exponent search on the device: (best_alpha [1] float64, losses [grid+1]
    float64), both device tensors, valid once the current stream is synchronised."""
    if w.dim() != 2 or x_cal.dim() != 2:
        raise ValueError("w must be [N, K] and x_cal [rows, K]")
    n, k = w.shape
    rows = x_cal.shape[0]
    if x_cal.shape[1] != k:
        raise ValueError("x_cal must be [rows, K] with the weights' K")
    _same_device(w, x_cal=x_cal, ws=ws)
    need = awq_scale_search_workspace_bytes(rows, n, k, group, fmt)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    losses = torch.empty(grid + 1, dtype=torch.float64, device=w.device)
    best = torch.empty(1, dtype=torch.float64, device=w.device)
    _check(lib().awq_scale_search(_dev(w, "w", torch.float16), _dev(x_cal, "x_cal", torch.float16),
                                  rows, n, k, group, fmt, grid, losses.data_ptr(),
                                  best.data_ptr(), _dev(ws, "ws", torch.uint8), ws.numel(),
                                  _stream(w.device)), "awq_scale_search")
    return best, losses


def awq_chain_state_bytes() -> int:
    return int(lib().awq_chain_state_bytes())


def chain_state(device) -> torch.Tensor:
    """A zeroed state buffer for awq_gemv_chain (one per stream that runs chains)."""
    return torch.zeros(awq_chain_state_bytes(), dtype=torch.uint8, device=device)


def chain_errors(state: torch.Tensor) -> int:
    """Waits that ran out in the chain calls since the state was last cleared (word 0;
    synchronises with the device)."""
    return int(state[:4].view(torch.int32).item())


def awq_gemv_chain(layers, state: torch.Tensor):
    """Run M = 1 products in one launch. `layers` is a list of dicts with keys packed, n,
    k and optionally x ([K] or [1, K] fp16; required when src is -1), inv_s_c, group,
    fmt, y ([N] or [1, N] fp16, allocated when absent) and src (index of an earlier
    layer whose output is this layer's input, default -1). Returns the outputs, [1, N]
    each."""
    n_layers = len(layers)
    if n_layers > CHAIN_MAX_LAYERS:
        raise ValueError(f"at most {CHAIN_MAX_LAYERS} layers per call")
    _dev(state, "state", torch.uint8)
    _at_least(state, "state", awq_chain_state_bytes())
    arr = (ChainLayer * max(n_layers, 1))()
    outs = []
    for i, spec in enumerate(layers):
        n, k = int(spec["n"]), int(spec["k"])
        group, fmt = int(spec.get("group", GROUP)), int(spec.get("fmt", FMT_ASYM))
        src = int(spec.get("src", -1))
        x, inv, packed, y = spec.get("x"), spec.get("inv_s_c"), spec["packed"], spec.get("y")
        if not -1 <= src < i:
            raise ValueError(f"layer {i}: src must be -1 or an earlier layer")
        if src >= 0:
            if int(layers[src]["n"]) != k:
                raise ValueError(f"layer {i}: its input (layer {src}) has N != K")
            x = None
        elif x is None:
            raise ValueError(f"layer {i}: x is required when src is -1")
        else:
            x = x.reshape(-1)
            _shape(x, f"layers[{i}].x", (k,))
        if y is None:
            y = torch.empty((1, n), dtype=torch.float16, device=state.device)
        _shape(y.reshape(-1), f"layers[{i}].y", (n,))
        _shape(inv, f"layers[{i}].inv_s_c", (k,))
        _at_least(packed, f"layers[{i}].packed", awq_repacked_bytes(n, k, group, fmt))
        _same_device(state, x=x, inv_s_c=inv, packed=packed, y=y)
        arr[i] = ChainLayer(_opt(x, "x", torch.float16), _opt(inv, "inv_s_c", torch.float16),
                            _dev(packed, "packed", torch.uint8), _dev(y, "y", torch.float16),
                            n, k, group, fmt, src, 0)
        outs.append(y.reshape(1, n))
    _check(lib().awq_gemv_chain(ctypes.cast(arr, _vp), n_layers, state.data_ptr(),
                                _stream(state.device)), "awq_gemv_chain")
    return outs


# --------------------------------------------------------------------- convenience

_WS = {}


def workspace(m: int, n: int, k: int, device, group: int = GROUP) -> torch.Tensor | None:
    """A workspace large enough for (m, n, k), cached per device and per stream and grown
    on demand (the library overwrites what it uses on every call, so no initialisation
    is needed). Calls that share a workspace must be ordered; keying the cache by the
    current stream keeps layers called on different streams on different buffers. A
    buffer replaced by a larger one goes back to PyTorch's caching allocator, which hands
    its memory out again only in the order of that stream."""
    need = awq_workspace_bytes(m, n, k, group)
    if need == 0:
        return None
    dev = torch.device(device)
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (dev.type, index, torch.cuda.current_stream(index).cuda_stream)
    cur = _WS.get(key)
    if cur is None or cur.numel() < need:
        cur = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device=dev)
        _WS[key] = cur
    return cur


class QuantLinear:
    """A quantized linear layer on the device: y = x . deq(Wq)^T.

    Built from fp16 weights with ``QuantLinear.from_weight`` (channel scale from
    calibration rows, fold, quantize, pack, repack -- all in the library's kernels).
    Calls go to awq_gemm, which runs the decode kernel itself where that is faster (a few
    rows, or up to 16 rows on small layers); ``gemv_max_m`` sends up to that many rows to
    awq_gemv directly instead.
    """

    def __init__(self, packed, n, k, inv_s_c=None, group=GROUP, fmt=FMT_ASYM, gemv_max_m=0):
        self.packed, self.n, self.k = packed, n, k
        self.inv_s_c, self.group, self.fmt = inv_s_c, group, fmt
        self.gemv_max_m = gemv_max_m

    @classmethod
    def from_weight(cls, w, x_cal=None, alpha=0.5, group=GROUP, fmt=FMT_ASYM, **kw):
        s_c = inv = None
        if x_cal is not None:
            s_c, inv = awq_channel_scale(x_cal, alpha)
        qweight, scales, qzeros = awq_pack(w, s_c, group, fmt)
        n, k = w.shape
        packed = awq_repack(qweight, scales, qzeros, n, k, group, fmt)
        return cls(packed, n, k, inv, group, fmt, **kw)

    def __call__(self, x, y=None):
        m = x.shape[0]
        ws = workspace(max(m, 1), self.n, self.k, x.device, self.group)
        fn = awq_gemv if 1 <= m <= self.gemv_max_m else awq_gemm
        return fn(x, self.inv_s_c, self.packed, self.n, self.k, self.group, self.fmt, y, ws)
