"""qmv_swiglu_quantize (SwiGLU of a gate+up output, quantized to Q8) and the
MoE FFN step it joins (gate+up routed matvec -> SwiGLU + Q8 -> route-weighted
down matvec), against the oracle.

The fp32 h = silu(g) * u of the GPU is compared with the oracle's fp64 h
within 4e-7 relative (a few fp32 roundings and the exp's own error), plus
3e-37 max(|u|, 1) absolute: for g < -88.7 exp(-g) overflows fp32 and silu(g) comes out
as -0, where its true magnitude is below 89 e^-88.7 < 3e-37.  The Q8
blocks are an integer decision taken from that fp32 h, so they are compared
bit-exactly with the oracle's quantization of the GPU's own h; each stage of
the FFN step is likewise checked with the GPU's output of the stage before
as the oracle's input."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y, gpu, need_gpu, quantize, say, to_dev, x_host

pytestmark = gpu

H_REL = 4e-7


def _check_swiglu(qmv, gu: np.ndarray, n_ff: int, what: str):
    rows = gu.shape[0]
    gu_d = to_dev(gu)
    h_d = torch.empty((rows, n_ff), dtype=torch.float32, device="cuda")
    xq = qmv.swiglu_quantize(gu_d, n_ff, h_out=h_d)
    h = h_d.cpu().numpy()
    h_ref = oracle.swiglu(gu, n_ff)
    err = np.abs(h.astype(np.float64) - h_ref)
    u = np.abs(gu[:, n_ff:2 * n_ff].astype(np.float64))
    bad = err > H_REL * np.abs(h_ref) + 3e-37 * np.maximum(np.abs(u), 1.0)
    assert not bad.any(), (what, np.argwhere(bad)[:3], h[bad][:3], h_ref[bad][:3])
    qs, d, s = qmv.act_fields(xq, rows, n_ff)
    qs_r, d_r, s_r = oracle.quantize_act(h)
    assert np.array_equal(qs.cpu().numpy(), qs_r), what
    assert np.array_equal(d.cpu().numpy(), d_r), what
    assert np.array_equal(s.cpu().numpy(), s_r), what
    return xq, h


def test_swiglu_moe_shape():
    """The gate+up output of 64 tokens x top-8 slots: 512 rows of 3072."""
    qmv = need_gpu()
    g = synth.make_x(512, 1536, "swiglu/g") * np.float32(3.0)
    u = synth.make_x(512, 1536, "swiglu/u")
    _check_swiglu(qmv, np.concatenate([g, u], 1), 1536, "512x1536")


def test_swiglu_edges():
    qmv = need_gpu()
    say("swiglu edges")
    n = 64
    g = np.zeros((5, n), np.float32)
    u = np.ones((5, n), np.float32)
    g[1] = np.linspace(-120.0, 120.0, n, dtype=np.float32)  # exp overflow on both sides
    g[2, :32] = 0.0
    u[2, :32] = 5.0  # a block that is exactly zero
    g[3] = 1.0
    u[3] = np.float32(-1.0)
    g[4] = synth.make_x(1, n, "swiglu/e")[0] * np.float32(20.0)
    u[4] = synth.make_x(1, n, "swiglu/f")[0] * np.float32(1e-3)
    gu = np.concatenate([g, u], 1)
    xq, h = _check_swiglu(qmv, gu, n, "edges")
    assert np.all(h[2, :32] == 0.0)
    # a wider row stride: the gate and up halves are read from their columns
    wide = np.concatenate([g, u, np.full((5, 32), 1e30, np.float32)], 1)
    _check_swiglu(qmv, wide, n, "ldg > 2 n_ff")
    # one row, one block
    _check_swiglu(qmv, gu[3:4, :][:, np.r_[0:32, 64:96]], 32, "1x32")


def test_moe_ffn_step():
    """x -> Q8 -> gate+up (one output per slot) -> SwiGLU + Q8 -> down with the
    route weights, on a small expert set; every stage against the oracle."""
    qmv = need_gpu()
    fmt, e_n, n_ff, k, top_k, t = synth.IQ4_XS, 6, 256, 256, 3, 5
    w_gu = synth.make_weights(fmt, e_n * 2 * n_ff, k, "ffn/gu").data
    w_dn = synth.make_weights(fmt, e_n * k, n_ff, "ffn/dn").data
    ids = np.array([[0, 4, 2], [5, 5, 1], [3, 0, 4], [2, 1, 0], [1, 3, 5]], np.int32)
    rw = synth.normal_f32(synth.stream("ffn/rw"), 0, t * top_k).reshape(t, top_k)
    x = x_host(t, k, "ffn/x")
    xq = quantize(qmv, x)
    ws = torch.zeros(qmv.moe_workspace_bytes(fmt, e_n, 2 * n_ff, k, t, top_k), dtype=torch.uint8,
                     device="cuda")
    y_gu = qmv.moe_matvec(fmt, to_dev(w_gu), e_n, 2 * n_ff, k, xq, False, to_dev(ids), None, ws)
    qs, d, s = oracle.quantize_act(x)
    yr, mag = oracle.moe_matvec(fmt, w_gu, e_n, 2 * n_ff, k, qs, d, s, ids, None, False)
    y_gu_h = y_gu.cpu().numpy()
    assert_y(y_gu_h, yr, mag, "gate+up")
    hq, h = _check_swiglu(qmv, y_gu_h.reshape(t * top_k, 2 * n_ff), n_ff, "ffn swiglu")
    ws2 = torch.zeros(qmv.moe_workspace_bytes(fmt, e_n, k, n_ff, t, top_k), dtype=torch.uint8,
                      device="cuda")
    y = qmv.moe_matvec(fmt, to_dev(w_dn), e_n, k, n_ff, hq, True, to_dev(ids), to_dev(rw), ws2)
    qs, d, s = oracle.quantize_act(h)
    yr, mag = oracle.moe_matvec(fmt, w_dn, e_n, k, n_ff, qs, d, s, ids, rw, True)
    assert_y(y.cpu().numpy(), yr, mag, "down")
