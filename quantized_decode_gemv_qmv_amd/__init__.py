"""Quantized decode matvec for AMD MI355X (gfx950).

Python binding of ``libqmv.so`` (the C ABI declared in ``include/qmv.h``).
This module only marshals arguments: every step of the computation runs in
the library's HIP kernels.  PyTorch supplies device memory and the stream; the
calls are enqueued on ``torch.cuda.current_stream()`` unless a stream is
given, and never synchronize.

If the library has not been built, importing works but the first call raises
``RuntimeError`` -- there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "Q8_0", "Q4_K", "IQ4_XS", "Q5_K", "Q6_K", "Q8G128", "QmvError", "lib", "library_path", "symbols",
    "row_bytes", "act_bytes", "act_offsets", "act_fields", "matvec_workspace_bytes",
    "moe_workspace_bytes", "quantize_act", "matvec", "matvec_x", "matvec_batch", "moe_matvec", "moe_matvec_noalloc",
    "moe_gate_up_swiglu",
    "block_dots",
    "block_dots_mx", "moe_block_dots", "stream_read",
    "set_tuning", "swiglu_quantize", "router_topk", "variant_name", "variants", "pick_variant", "matvec_plan", "MAX_TOKENS", "MAX_MOE_TOKENS",
]

Q8_0, Q4_K, IQ4_XS, Q5_K, Q6_K, Q8G128 = 0, 1, 2, 3, 4, 5
MAX_TOKENS = 16
MAX_MOE_TOKENS = 64
MAX_BATCH = 8

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
_LIB = os.path.join(_PKG, "libqmv.so")
_HEADER = os.path.join(_ROOT, "include", "qmv.h")
_lib = None


class _Item(ctypes.Structure):
    """qmv_matvec_item of include/qmv.h."""
    _fields_ = [("w", ctypes.c_void_p), ("n_rows", ctypes.c_int64), ("y", ctypes.c_void_p),
                ("ldy", ctypes.c_int64), ("residual", ctypes.c_void_p), ("ldr", ctypes.c_int64)]


class QmvError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _lib.qmv_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg}")
        self.status = status


def library_path() -> str:
    return _LIB


def symbols() -> list[str]:
    """Function names declared in include/qmv.h."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_\w+)\s*\(", text)))


def lib():
    """The loaded library; raises if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        raise RuntimeError(f"{_LIB} is missing: build it with __graft_entry__.build() "
                           "(or python quantized_decode_gemv_qmv_amd/build.py)")
    L = ctypes.CDLL(_LIB)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "qmv_abi_version": ([], I),
        "qmv_last_hip_error": ([], I),
        "qmv_last_hip_error_name": ([], ctypes.c_char_p),
        "qmv_status_string": ([I], ctypes.c_char_p),
        "qmv_row_bytes": ([I, I64], SZ),
        "qmv_act_bytes": ([I64, I64], SZ),
        "qmv_act_offset_d": ([I64, I64], SZ),
        "qmv_act_offset_s": ([I64, I64], SZ),
        "qmv_quantize_act": ([P, I64, I64, I64, P, P], I),
        "qmv_swiglu_quantize": ([P, I64, I64, I64, P, P, P], I),
        "qmv_router_topk": ([P, I64, I64, I64, P, I64, I64, P, P, P, P, P], I),
        "qmv_matvec_workspace_bytes": ([I, I64, I64, I64], SZ),
        "qmv_matvec": ([I, P, I64, I64, P, I64, P, I64, P, SZ, P], I),
        "qmv_matvec_batch": ([I, ctypes.POINTER(_Item), I64, I64, P, I64, P], I),
        "qmv_matvec_x": ([I, P, I64, I64, P, I64, I64, P, I64, P, P, SZ, P], I),
        "qmv_moe_workspace_bytes": ([I, I64, I64, I64, I64, I64], SZ),
        "qmv_moe_matvec": ([I, P, I64, I64, I64, P, I, P, P, I64, I64, P, P, SZ, P], I),
        "qmv_moe_matvec_noalloc": ([I, P, I64, I64, I64, P, I, P, P, I64, I64, P, P], I),
        "qmv_moe_gate_up_swiglu": ([I, P, I64, I64, I64, P, P, I64, I64, P, P, P, SZ, P], I),
        "qmv_block_dots": ([I, P, I64, I64, P, I64, P, P], I),
        "qmv_block_dots_mx": ([I, P, I64, I64, P, I64, I64, I, P, P], I),
        "qmv_moe_block_dots": ([I, P, I64, I64, I64, P, I, P, I64, I64, I64, P, P, SZ, P], I),
        "qmv_stream_read": ([P, I64, P, P], I),
        "qmv_set_tuning": ([ctypes.c_char_p, I64], I),
        "qmv_variant_name": ([I64], ctypes.c_char_p),
        "qmv_pick_variant": ([I, I64, I64, I64], I64),
        "qmv_matvec_plan": ([I, I64, I64, I64, I, ctypes.POINTER(I64), ctypes.POINTER(I)], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


# ------------------------------------------------------------------ helpers
def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        if status == 5:  # QMV_ERR_HIP: name the runtime's error
            what = f"{what} ({lib().qmv_last_hip_error_name().decode()})"
        raise QmvError(status, what)


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")


# ------------------------------------------------------------------- sizes
def row_bytes(fmt: int, k: int) -> int:
    return int(lib().qmv_row_bytes(fmt, k))


def act_bytes(n_tok: int, k: int) -> int:
    return int(lib().qmv_act_bytes(n_tok, k))


def act_offsets(n_tok: int, k: int) -> tuple[int, int]:
    L = lib()
    return int(L.qmv_act_offset_d(n_tok, k)), int(L.qmv_act_offset_s(n_tok, k))


def act_fields(xq: torch.Tensor, n_tok: int, k: int):
    """Views (qs int8 [T][K], d fp32 [T][K/32], s int32 [T][K/32]) of a Q8
    activation buffer."""
    od, os_ = act_offsets(n_tok, k)
    nb = k // 32
    qs = xq[: n_tok * k].view(torch.int8).view(n_tok, k)
    d = xq[od: od + 4 * n_tok * nb].view(torch.float32).view(n_tok, nb)
    s = xq[os_: os_ + 4 * n_tok * nb].view(torch.int32).view(n_tok, nb)
    return qs, d, s


def swiglu_quantize(gu: torch.Tensor, n_ff: int, out: torch.Tensor | None = None,
                    h_out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """gu fp32 [R][>= 2 n_ff] (gate | up) -> Q8 activation buffer of
    h = silu(gate) * up [R][n_ff]; h_out (fp32 [R][n_ff]) receives h."""
    _need(gu, torch.float32, "gu")
    if gu.dim() != 2 or gu.stride(1) != 1:
        raise ValueError("gu must be a 2-D tensor with unit column stride")
    rows = gu.shape[0]
    if out is None:
        out = torch.empty(act_bytes(rows, n_ff), dtype=torch.uint8, device=gu.device)
    if h_out is not None:
        _need(h_out, torch.float32, "h_out")
    ldg = gu.stride(0) if rows > 1 else gu.shape[1]  # a single row's stride is arbitrary
    _check(lib().qmv_swiglu_quantize(_ptr(gu), ldg, rows, n_ff, _ptr(out), _ptr(h_out),
                                     _stream(stream)), "qmv_swiglu_quantize")
    return out


def router_topk(x: torch.Tensor, wr: torch.Tensor, top_k: int, ids: torch.Tensor | None = None,
                weights: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                xq: torch.Tensor | None = None, stream=None):
    """x fp32 [T][K], router weights fp32 [E][K] -> (ids int32 [T][top_k],
    weights fp32 [T][top_k]); logits (fp32 [T][E], allocated when None)
    receives the router logits, xq (optional) the Q8 blocks of x.  x may
    have a row stride beyond K (a multiple of 4)."""
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dtype != torch.float32 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a float32 CUDA tensor with unit column stride")
    _need(wr, torch.float32, "wr")
    n_tok, k = x.shape
    e = wr.shape[0]
    if ids is None:
        ids = torch.empty((n_tok, top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((n_tok, top_k), dtype=torch.float32, device=x.device)
    if logits is None:
        logits = torch.empty((n_tok, e), dtype=torch.float32, device=x.device)
    _need(logits, torch.float32, "logits")
    ldx = x.stride(0) if n_tok > 1 else k
    if xq is not None:
        _need(xq, torch.uint8, "xq")
        if xq.numel() < act_bytes(n_tok, k):
            raise ValueError("activation buffer too small")
    _check(lib().qmv_router_topk(_ptr(x), ldx, n_tok, k, _ptr(wr), e, top_k, _ptr(ids), _ptr(weights),
                                 _ptr(logits), _ptr(xq), _stream(stream)), "qmv_router_topk")
    return ids, weights


def matvec_workspace_bytes(fmt: int, n_rows: int, k: int, n_tok: int) -> int:
    return int(lib().qmv_matvec_workspace_bytes(fmt, n_rows, k, n_tok))


def moe_workspace_bytes(fmt: int, n_experts: int, n_rows: int, k: int, n_tok: int,
                        top_k: int) -> int:
    return int(lib().qmv_moe_workspace_bytes(fmt, n_experts, n_rows, k, n_tok, top_k))


# --------------------------------------------------------------- entry points
def quantize_act(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """x fp32 [T][K] (row stride >= K) -> Q8 activation buffer (uint8)."""
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dtype != torch.float32 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a float32 CUDA tensor with unit column stride")
    n_tok, k = x.shape
    nbytes = act_bytes(n_tok, k)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    if out.numel() < nbytes:
        raise ValueError("activation buffer too small")
    ldx = x.stride(0) if n_tok > 1 else k  # a single row's stride is arbitrary
    _check(lib().qmv_quantize_act(_ptr(x), ldx, n_tok, k, _ptr(out), _stream(stream)),
           "qmv_quantize_act")
    return out


def matvec(fmt: int, w: torch.Tensor, n_rows: int, k: int, xq: torch.Tensor, n_tok: int,
           y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """y fp32 [T][N] = W xq.  ``ws`` (uint8, zero-filled once) enables split-K."""
    _need(w, torch.uint8, "w")
    _need(xq, torch.uint8, "xq")
    if y is None:
        y = torch.empty((n_tok, n_rows), dtype=torch.float32, device=w.device)
    if y.dtype != torch.float32 or not y.is_cuda or y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be a float32 CUDA tensor [T][ldy] with unit column stride")
    if w.numel() < n_rows * row_bytes(fmt, k):
        raise ValueError("w holds fewer than n_rows rows")
    wsz = 0 if ws is None else ws.numel()
    if ws is not None:
        _need(ws, torch.uint8, "ws")
    ldy = y.stride(0) if y.shape[0] > 1 else y.shape[1]
    _check(lib().qmv_matvec(fmt, _ptr(w), n_rows, k, _ptr(xq), n_tok, _ptr(y), ldy,
                            _ptr(ws), wsz, _stream(stream)), "qmv_matvec")
    return y


def matvec_x(fmt: int, w: torch.Tensor, n_rows: int, k: int, x: torch.Tensor,
             xq: torch.Tensor | None = None, y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
             stream=None):
    """The decode step from fp32 x [T][K]: (y [T][N] = W Q8(x), xq = Q8(x)).
    One launch for one or two tokens (the matvec quantizes x itself)."""
    _need(w, torch.uint8, "w")
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dtype != torch.float32 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a float32 CUDA tensor with unit column stride")
    n_tok = x.shape[0]
    if xq is None:
        xq = torch.empty(act_bytes(n_tok, k), dtype=torch.uint8, device=x.device)
    _need(xq, torch.uint8, "xq")
    if y is None:
        y = torch.empty((n_tok, n_rows), dtype=torch.float32, device=w.device)
    if y.dtype != torch.float32 or not y.is_cuda or y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be a float32 CUDA tensor [T][ldy] with unit column stride")
    if w.numel() < n_rows * row_bytes(fmt, k):
        raise ValueError("w holds fewer than n_rows rows")
    if ws is not None:
        _need(ws, torch.uint8, "ws")
    _check(lib().qmv_matvec_x(fmt, _ptr(w), n_rows, k, _ptr(x), _ld(x), n_tok, _ptr(y), _ld(y), _ptr(xq),
                              _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "qmv_matvec_x")
    return y, xq


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]  # a single row's stride is arbitrary


def matvec_batch(fmt: int, items, k: int, xq: torch.Tensor, n_tok: int, stream=None) -> list:
    """Sibling matvecs over one activation buffer in one launch.  ``items`` is
    a sequence of (w, n_rows, y, residual): y (fp32 [T][>= n_rows], allocated
    when None) receives W xq, plus residual (fp32 [T][>= n_rows]) when it is
    not None; residual may be y itself.  Returns the list of y."""
    _need(xq, torch.uint8, "xq")
    arr = (_Item * max(1, len(items)))()
    outs = []
    for i, (w, n_rows, y, res) in enumerate(items):
        _need(w, torch.uint8, "w")
        if w.numel() < n_rows * row_bytes(fmt, k):
            raise ValueError("w holds fewer than n_rows rows")
        if y is None:
            y = torch.empty((n_tok, n_rows), dtype=torch.float32, device=w.device)
        for name, t in (("y", y), ("residual", res)):
            if t is not None and (t.dtype != torch.float32 or not t.is_cuda or t.dim() != 2
                                  or t.stride(1) != 1):
                raise ValueError(f"{name} must be a float32 CUDA tensor [T][ld] with unit column stride")
        arr[i] = _Item(w.data_ptr(), n_rows, y.data_ptr(), _ld(y),
                       None if res is None else res.data_ptr(), 0 if res is None else _ld(res))
        outs.append(y)
    _check(lib().qmv_matvec_batch(fmt, arr, len(items), k, _ptr(xq), n_tok, _stream(stream)),
           "qmv_matvec_batch")
    return outs


def moe_matvec(fmt: int, w: torch.Tensor, n_experts: int, n_rows: int, k: int,
               xq: torch.Tensor, x_per_slot: bool, ids: torch.Tensor,
               route_w: torch.Tensor | None, ws: torch.Tensor,
               y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Expert-grouped routed matvec.  route_w None -> y [T][top_k][N];
    else y [T][N] = sum_s route_w[t][s] * W[ids[t][s]] x."""
    _need(w, torch.uint8, "w")
    _need(xq, torch.uint8, "xq")
    _need(ids, torch.int32, "ids")
    _need(ws, torch.uint8, "ws")
    n_tok, top_k = ids.shape
    if route_w is not None:
        _need(route_w, torch.float32, "route_w")
        if tuple(route_w.shape) != (n_tok, top_k):
            raise ValueError("route_w must match ids")
    shape = (n_tok, n_rows) if route_w is not None else (n_tok, top_k, n_rows)
    if y is None:
        y = torch.empty(shape, dtype=torch.float32, device=w.device)
    _need(y, torch.float32, "y")
    if y.numel() < n_tok * n_rows * (1 if route_w is not None else top_k):
        raise ValueError("y too small")
    if w.numel() < n_experts * n_rows * row_bytes(fmt, k):
        raise ValueError("w holds fewer than n_experts * n_rows rows")
    _check(lib().qmv_moe_matvec(fmt, _ptr(w), n_experts, n_rows, k, _ptr(xq), int(bool(x_per_slot)),
                                _ptr(ids), _ptr(route_w), n_tok, top_k, _ptr(y), _ptr(ws),
                                ws.numel(), _stream(stream)), "qmv_moe_matvec")
    return y


def moe_gate_up_swiglu(fmt: int, w: torch.Tensor, n_experts: int, n_ff: int, k: int, xq: torch.Tensor,
                       ids: torch.Tensor, ws: torch.Tensor, hq: torch.Tensor | None = None,
                       gu: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Routed gate+up (2 n_ff rows per expert, gate first) with SwiGLU and
    Q8 folded in: returns hq, the Q8 activation buffer of the n_tok * top_k
    slot rows of h; gu (fp32 [T][top_k][2 n_ff]), if given, receives the
    gate+up outputs."""
    _need(w, torch.uint8, "w")
    _need(xq, torch.uint8, "xq")
    _need(ids, torch.int32, "ids")
    _need(ws, torch.uint8, "ws")
    n_tok, top_k = ids.shape
    if hq is None:
        hq = torch.empty(act_bytes(n_tok * top_k, n_ff), dtype=torch.uint8, device=w.device)
    _need(hq, torch.uint8, "hq")
    if hq.numel() < act_bytes(n_tok * top_k, n_ff):
        raise ValueError("hq too small")
    if gu is not None:
        _need(gu, torch.float32, "gu")
        if gu.numel() < n_tok * top_k * 2 * n_ff:
            raise ValueError("gu too small")
    if w.numel() < n_experts * 2 * n_ff * row_bytes(fmt, k):
        raise ValueError("w holds fewer than n_experts * 2 n_ff rows")
    _check(lib().qmv_moe_gate_up_swiglu(fmt, _ptr(w), n_experts, n_ff, k, _ptr(xq), _ptr(ids), n_tok, top_k,
                                        _ptr(hq), _ptr(gu), _ptr(ws), ws.numel(), _stream(stream)),
           "qmv_moe_gate_up_swiglu")
    return hq


def moe_matvec_noalloc(fmt: int, w: torch.Tensor, n_experts: int, n_rows: int, k: int,
                       xq: torch.Tensor, x_per_slot: bool, ids: torch.Tensor,
                       route_w: torch.Tensor | None, y: torch.Tensor, stream=None) -> torch.Tensor:
    """moe_matvec on the library's device-resident workspace (no caller
    workspace; y must be given, so that nothing is allocated)."""
    _need(w, torch.uint8, "w")
    _need(xq, torch.uint8, "xq")
    _need(ids, torch.int32, "ids")
    _need(y, torch.float32, "y")
    n_tok, top_k = ids.shape
    if route_w is not None:
        _need(route_w, torch.float32, "route_w")
        if tuple(route_w.shape) != (n_tok, top_k):
            raise ValueError("route_w must match ids")
    if y.numel() < n_tok * n_rows * (1 if route_w is not None else top_k):
        raise ValueError("y too small")
    if w.numel() < n_experts * n_rows * row_bytes(fmt, k):
        raise ValueError("w holds fewer than n_experts * n_rows rows")
    _check(lib().qmv_moe_matvec_noalloc(fmt, _ptr(w), n_experts, n_rows, k, _ptr(xq), int(bool(x_per_slot)),
                                        _ptr(ids), _ptr(route_w), n_tok, top_k, _ptr(y), _stream(stream)),
           "qmv_moe_matvec_noalloc")
    return y


def block_dots(fmt: int, w: torch.Tensor, n_rows: int, k: int, xq: torch.Tensor, n_tok: int,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Exact integer partial of every 32-block: int32 [T][N][K/32][c]."""
    _need(w, torch.uint8, "w")
    _need(xq, torch.uint8, "xq")
    nc = 2 if fmt in (Q4_K, Q5_K) else 1
    if out is None:
        out = torch.empty((n_tok, n_rows, k // 32, nc), dtype=torch.int32, device=w.device)
    _need(out, torch.int32, "out")
    _check(lib().qmv_block_dots(fmt, _ptr(w), n_rows, k, _ptr(xq), n_tok, _ptr(out),
                                _stream(stream)), "qmv_block_dots")
    return out


def block_dots_mx(fmt: int, w: torch.Tensor, n_rows: int, k: int, xq: torch.Tensor, n_tok: int,
                  variant: int = -1, slices: int = 0, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """The block integers of block_dots, computed by the matrix-core kernel
    (variant -1: the one qmv_matvec runs; slices 0 unsplit, -1 automatic,
    n >= 2 forced): int32 [T][N][K/32][c]."""
    _need(w, torch.uint8, "w")
    _need(xq, torch.uint8, "xq")
    nc = 2 if fmt == Q4_K else 1
    if out is None:
        out = torch.empty((n_tok, n_rows, k // 32, nc), dtype=torch.int32, device=w.device)
    _need(out, torch.int32, "out")
    if out.numel() < n_tok * n_rows * (k // 32) * nc:
        raise ValueError("out too small")
    _check(lib().qmv_block_dots_mx(fmt, _ptr(w), n_rows, k, _ptr(xq), n_tok, variant, slices, _ptr(out),
                                   _stream(stream)), "qmv_block_dots_mx")
    return out


def moe_block_dots(fmt: int, w: torch.Tensor, n_experts: int, n_rows: int, k: int, xq: torch.Tensor,
                   x_per_slot: bool, ids: torch.Tensor, ws: torch.Tensor, slot_rows: int = 0,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The block integers of every routed slot from the matrix-core MoE
    kernel: int32 [T * top_k][N][K/32][c] (dropped slots' entries untouched)."""
    _need(w, torch.uint8, "w")
    _need(xq, torch.uint8, "xq")
    _need(ids, torch.int32, "ids")
    _need(ws, torch.uint8, "ws")
    n_tok, top_k = ids.shape
    nc = 2 if fmt == Q4_K else 1
    if out is None:
        out = torch.zeros((n_tok * top_k, n_rows, k // 32, nc), dtype=torch.int32, device=w.device)
    _need(out, torch.int32, "out")
    if out.numel() < n_tok * top_k * n_rows * (k // 32) * nc:
        raise ValueError("out too small")
    if w.numel() < n_experts * n_rows * row_bytes(fmt, k):
        raise ValueError("w holds fewer than n_experts * n_rows rows")
    _check(lib().qmv_moe_block_dots(fmt, _ptr(w), n_experts, n_rows, k, _ptr(xq), int(bool(x_per_slot)),
                                    _ptr(ids), n_tok, top_k, slot_rows, _ptr(out), _ptr(ws), ws.numel(),
                                    _stream(stream)), "qmv_moe_block_dots")
    return out


def stream_read(t: torch.Tensor, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Read every byte of t once (the plain-read ceiling of a weight stream)."""
    _need(t, torch.uint8, "t")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=t.device)
    _need(sink, torch.int32, "sink")
    _check(lib().qmv_stream_read(_ptr(t), t.numel(), _ptr(sink), _stream(stream)), "qmv_stream_read")
    return sink


# ------------------------------------------------------------------ tuning
def set_tuning(key: str, value: int) -> None:
    _check(lib().qmv_set_tuning(key.encode(), int(value)), f"qmv_set_tuning({key})")


def variant_name(index: int) -> str | None:
    r = lib().qmv_variant_name(index)
    return None if r is None else r.decode()


def variants() -> list[str]:
    out, i = [], 0
    while (n := variant_name(i)) is not None:
        out.append(n)
        i += 1
    return out


def pick_variant(fmt: int, n_rows: int, k: int, n_tok: int) -> int:
    return int(lib().qmv_pick_variant(fmt, n_rows, k, n_tok))


def matvec_plan(fmt: int, n_rows: int, k: int, n_tok: int, with_workspace: bool) -> tuple[int, int]:
    """(kernel variant, K slices over workgroups) qmv_matvec would run."""
    v, s = ctypes.c_int64(), ctypes.c_int()
    _check(lib().qmv_matvec_plan(fmt, n_rows, k, n_tok, int(with_workspace), ctypes.byref(v), ctypes.byref(s)),
           "qmv_matvec_plan")
    return int(v.value), int(s.value)
