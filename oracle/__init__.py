"""CPU oracle for the quantized decode matvec -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg
may import this package.  The product path (the HIP library and its binding)
never calls it; the two share no code.

The arithmetic lives in ``qmv_oracle.c`` (plain scalar C, fp64 terms, OpenMP
over output rows only); this module is ctypes marshalling over numpy arrays.
The library is built with gcc on first use if it is not there yet; ``build()``
rebuilds it unconditionally.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB = os.path.join(_HERE, "liboqmv.so")

Q8_0, Q4_K, IQ4_XS, Q5_K, Q6_K, Q8G128 = 0, 1, 2, 3, 4, 5
_lib = None


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_row_bytes.argtypes = [I, I64]
    lib.oracle_row_bytes.restype = I64
    lib.oracle_unpack.argtypes = [I, P, I64, I64, P, P, P, P, P]
    lib.oracle_dequant.argtypes = [I, P, I64, I64, P]
    lib.oracle_quantize_act.argtypes = [P, I64, I64, I64, P, P, P]
    lib.oracle_block_dots.argtypes = [I, P, I64, I64, P, P, I64, P]
    lib.oracle_matvec.argtypes = [I, P, I64, I64, P, P, P, I64, P, P]
    lib.oracle_matvec_residual.argtypes = [I, P, I64, I64, P, P, P, I64, P, I64, P, P]
    lib.oracle_moe_matvec.argtypes = [I, P, I64, I64, I64, P, P, P, I, P, P, I64, I64, P, P]
    lib.oracle_swiglu.argtypes = [P, I64, I64, I64, P]
    lib.oracle_router_topk.argtypes = [P, I64, I64, I64, P, I64, I64, P, P, P]
    lib.oracle_topk_from_logits.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_threads.restype = I
    lib.oracle_set_threads.argtypes = [I]
    for f in ("oracle_unpack", "oracle_dequant", "oracle_quantize_act", "oracle_block_dots",
              "oracle_matvec", "oracle_matvec_residual", "oracle_moe_matvec", "oracle_swiglu", "oracle_router_topk",
              "oracle_topk_from_logits"):
        getattr(lib, f).restype = I
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected the arguments")


def row_bytes(fmt: int, k: int) -> int:
    return int(_load().oracle_row_bytes(fmt, k))


def threads() -> int:
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _w2d(fmt, w, k):
    w = np.ascontiguousarray(w, dtype=np.uint8)
    rb = row_bytes(fmt, k)
    if rb <= 0 or w.size % rb:
        raise ValueError("weight bytes do not hold whole rows")
    return w.reshape(-1, rb)


def unpack(fmt: int, w: np.ndarray, k: int) -> dict:
    w = _w2d(fmt, w, k)
    n = w.shape[0]
    nsb = k // 32 if fmt == Q8_0 else (k // 128 if fmt == Q8G128 else k // 256)
    d = np.zeros((n, nsb))
    dmin = np.zeros((n, nsb))
    nsc = 16 if fmt == Q6_K else 8  # q6_K: one scale per 16 weights
    sc = np.zeros((n, nsb, nsc), dtype=np.int32)
    m = np.zeros((n, nsb, 8), dtype=np.int32)
    q = np.zeros((n, k), dtype=np.int32)
    _check(_load().oracle_unpack(fmt, _p(w), n, k, _p(d), _p(dmin), _p(sc), _p(m), _p(q)))
    return dict(d=d, dmin=dmin, sc=sc, m=m, q=q)


def dequant(fmt: int, w: np.ndarray, k: int) -> np.ndarray:
    w = _w2d(fmt, w, k)
    out = np.zeros((w.shape[0], k))
    _check(_load().oracle_dequant(fmt, _p(w), w.shape[0], k, _p(out)))
    return out


def quantize_act(x: np.ndarray):
    """x fp32 [T][K] -> (qs int8 [T][K], d fp32 [T][K/32], s int32 [T][K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    t, k = x.shape
    qs = np.zeros((t, k), dtype=np.int8)
    d = np.zeros((t, k // 32), dtype=np.float32)
    s = np.zeros((t, k // 32), dtype=np.int32)
    _check(_load().oracle_quantize_act(_p(x), k, t, k, _p(qs), _p(d), _p(s)))
    return qs, d, s


def block_dots(fmt: int, w: np.ndarray, k: int, qs: np.ndarray, s: np.ndarray) -> np.ndarray:
    """int32 [T][N][K/32][c], c = 2 for q4_K and q5_K (A, B) else 1."""
    w = _w2d(fmt, w, k)
    qs = np.ascontiguousarray(qs, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.int32)
    t = qs.shape[0]
    nc = 2 if fmt in (Q4_K, Q5_K) else 1
    out = np.zeros((t, w.shape[0], k // 32, nc), dtype=np.int32)
    _check(_load().oracle_block_dots(fmt, _p(w), w.shape[0], k, _p(qs), _p(s), t, _p(out)))
    return out


def matvec(fmt: int, w: np.ndarray, k: int, qs, d, s, residual: np.ndarray | None = None):
    """(y, mag) fp64 [T][N]: y the reference output, mag the sum of |terms|.
    With a residual (fp32 [T][N]) it is one more term: y + r, mag + |r|."""
    w = _w2d(fmt, w, k)
    qs = np.ascontiguousarray(qs, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.int32)
    t = qs.shape[0]
    y = np.zeros((t, w.shape[0]))
    mag = np.zeros((t, w.shape[0]))
    if residual is None:
        _check(_load().oracle_matvec(fmt, _p(w), w.shape[0], k, _p(qs), _p(d), _p(s), t, _p(y), _p(mag)))
    else:
        r = np.ascontiguousarray(residual, dtype=np.float32)
        assert r.shape == (t, w.shape[0])
        _check(_load().oracle_matvec_residual(fmt, _p(w), w.shape[0], k, _p(qs), _p(d), _p(s), t, _p(r),
                                              r.shape[1], _p(y), _p(mag)))
    return y, mag


def moe_matvec(fmt: int, w: np.ndarray, n_experts: int, n_rows: int, k: int, qs, d, s,
               ids: np.ndarray, rw: np.ndarray | None, x_per_slot: bool):
    """Expert-routed matvec.  rw None -> (y, mag) [T][top_k][N]; else [T][N]."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    assert w.size == n_experts * n_rows * row_bytes(fmt, k)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    t, top_k = ids.shape
    qs = np.ascontiguousarray(qs, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.int32)
    assert qs.shape[0] == (t * top_k if x_per_slot else t)
    if rw is not None:
        rw = np.ascontiguousarray(rw, dtype=np.float32)
        shape = (t, n_rows)
    else:
        shape = (t, top_k, n_rows)
    y = np.zeros(shape)
    mag = np.zeros(shape)
    _check(_load().oracle_moe_matvec(fmt, _p(w), n_experts, n_rows, k, _p(qs), _p(d), _p(s),
                                     int(bool(x_per_slot)), _p(ids), _p(rw), t, top_k, _p(y), _p(mag)))
    return y, mag


def swiglu(gu: np.ndarray, n_ff: int) -> np.ndarray:
    """gu fp32 [R][>= 2 n_ff] (gate | up) -> h fp64 [R][n_ff] = silu(g) * u."""
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    if gu.ndim == 1:
        gu = gu[None]
    r, ld = gu.shape
    h = np.zeros((r, n_ff), dtype=np.float64)
    _check(_load().oracle_swiglu(_p(gu), ld, r, n_ff, _p(h)))
    return h


def router_topk(x: np.ndarray, wr: np.ndarray, top_k: int):
    """x fp32 [T][K], router weights fp32 [E][K] -> (ids int32 [T][top_k],
    w fp64 [T][top_k], logits fp64 [T][E])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    t, k = x.shape
    e = wr.shape[0]
    assert wr.shape == (e, k)
    ids = np.zeros((t, top_k), np.int32)
    w = np.zeros((t, top_k), np.float64)
    logits = np.zeros((t, e), np.float64)
    _check(_load().oracle_router_topk(_p(x), k, t, k, _p(wr), e, top_k, _p(ids), _p(w), _p(logits)))
    return ids, w, logits


def topk_from_logits(logits: np.ndarray, top_k: int):
    """fp32 logits [T][E] -> (ids int32 [T][top_k], w fp64 [T][top_k]) by the
    same selection and normalization as router_topk."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    t, e = logits.shape
    ids = np.zeros((t, top_k), np.int32)
    w = np.zeros((t, top_k), np.float64)
    _check(_load().oracle_topk_from_logits(_p(logits), t, e, top_k, _p(ids), _p(w)))
    return ids, w
