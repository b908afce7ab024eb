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


def _same_q8(qmv, a, b, rows, n):
    """Two Q8 buffers of (rows, n) hold the same quants, scales and sums (the
    alignment padding between the fields is written by neither path)."""
    return all(torch.equal(x_, y_) for x_, y_ in zip(qmv.act_fields(a, rows, n), qmv.act_fields(b, rows, n)))


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


E_C4, TOPK_C4, NFF_C4, K_C4 = 128, 8, 1536, 4096


@pytest.fixture(scope="module")
def c4_experts():
    need_gpu()
    from gpu_util import weights
    say("FFN: generating the 128-expert gate+up and down tensors")
    gu = weights(synth.IQ4_XS, E_C4 * 2 * NFF_C4, K_C4, "ffn_c4/gate_up")
    dn = weights(synth.IQ4_XS, E_C4 * K_C4, NFF_C4, "ffn_c4/down")
    return gu, dn


def _experts_host(w_dev, n_rows, used):
    """Host bytes of the experts in `used` ([len(used) * n_rows][row_bytes]) and
    the id map onto them."""
    rb = w_dev.shape[1]
    v = w_dev.view(E_C4, n_rows, rb)
    idx = torch.tensor(used, dtype=torch.int64, device="cuda")
    return v.index_select(0, idx).reshape(len(used) * n_rows, rb).cpu().numpy()


@pytest.mark.parametrize("t", [1, 6, 16, 64])
def test_moe_ffn_chain_workload(c4_experts, t):
    """The MoE FFN step at the workload's shape (128 IQ4_XS experts, gate+up
    3072 x 4096, down 4096 x 1536, top-8) through the library's own chain:
    router + top-k (writing Q8(x)) -> fused gate+up + SwiGLU + Q8 -> down with
    the router's weights.  Each stage is checked against the oracle with the
    GPU's previous stage as its input (the router's picks against the
    oracle's selection from the GPU logits; gate+up on every row of the
    routed experts; the Q8 blocks of h bit-exactly against the oracle's
    quantization of h from the GPU gate+up output; down within tolerance),
    and the fused launch's outputs bit-identical to the two-launch path."""
    qmv = need_gpu()
    gu_w, dn_w = c4_experts
    fmt = synth.IQ4_XS
    x = x_host(t, K_C4, "ffn_c4/x")
    wr = synth.make_x(E_C4, K_C4, "ffn_c4/router") * np.float32(1.0 / 64.0)
    x_d, wr_d = to_dev(x), to_dev(wr)
    xq = torch.empty(qmv.act_bytes(t, K_C4), dtype=torch.uint8, device="cuda")
    logits = torch.empty((t, E_C4), dtype=torch.float32, device="cuda")
    say(f"FFN chain T={t}: router")
    ids_d, rw_d = qmv.router_topk(x_d, wr_d, TOPK_C4, logits=logits, xq=xq)
    ids = ids_d.cpu().numpy()
    ids_r, w_r = oracle.topk_from_logits(logits.cpu().numpy(), TOPK_C4)
    assert np.array_equal(ids, ids_r)
    assert np.allclose(rw_d.cpu().numpy(), w_r, rtol=1e-5, atol=1e-7)
    qs, d, s = oracle.quantize_act(x)
    g_qs, g_d, g_s = (a_.cpu().numpy() for a_ in qmv.act_fields(xq, t, K_C4))
    assert np.array_equal(g_qs, qs) and np.array_equal(g_d, d) and np.array_equal(g_s, s)

    say(f"FFN chain T={t}: fused gate+up + SwiGLU + Q8")
    ws = torch.zeros(qmv.moe_workspace_bytes(fmt, E_C4, 2 * NFF_C4, K_C4, t, TOPK_C4), dtype=torch.uint8,
                     device="cuda")
    gu = torch.empty((t, TOPK_C4, 2 * NFF_C4), dtype=torch.float32, device="cuda")
    hq = qmv.moe_gate_up_swiglu(fmt, gu_w, E_C4, NFF_C4, K_C4, xq, ids_d, ws, gu=gu)
    hq_nogu = qmv.moe_gate_up_swiglu(fmt, gu_w, E_C4, NFF_C4, K_C4, xq, ids_d, ws)
    # the two-launch path
    gu2 = qmv.moe_matvec(fmt, gu_w, E_C4, 2 * NFF_C4, K_C4, xq, False, ids_d, None, ws)
    hq2 = qmv.swiglu_quantize(gu2.view(t * TOPK_C4, 2 * NFF_C4), NFF_C4)
    assert torch.equal(gu, gu2), "fused gate+up differs from the routed matvec"
    assert _same_q8(qmv, hq, hq2, t * TOPK_C4, NFF_C4), "fused Q8(h) differs"
    assert _same_q8(qmv, hq_nogu, hq2, t * TOPK_C4, NFF_C4), "fused Q8(h) without gu differs"
    used = sorted(set(ids.reshape(-1).tolist()))
    remap = np.vectorize({ex: i for i, ex in enumerate(used)}.get)(ids).astype(np.int32)
    gu_h = gu.cpu().numpy()
    yr, mag = oracle.moe_matvec(fmt, _experts_host(gu_w, 2 * NFF_C4, used), len(used), 2 * NFF_C4, K_C4,
                                qs, d, s, remap, None, False)
    assert_y(gu_h, yr, mag, f"gate+up T={t}")
    h_ref = oracle.swiglu(gu_h.reshape(t * TOPK_C4, 2 * NFF_C4), NFF_C4)
    hq_qs, hq_d, hq_s = (a_.cpu().numpy() for a_ in qmv.act_fields(hq, t * TOPK_C4, NFF_C4))
    # the blocks from the GPU's fp32 h (the oracle's fp64 h agrees within H_REL)
    h_gpu = torch.empty((t * TOPK_C4, NFF_C4), dtype=torch.float32, device="cuda")
    qmv.swiglu_quantize(gu.view(t * TOPK_C4, 2 * NFF_C4), NFF_C4, h_out=h_gpu)
    h_gpu = h_gpu.cpu().numpy()
    u_abs = np.abs(gu_h.reshape(t * TOPK_C4, 2 * NFF_C4)[:, NFF_C4:].astype(np.float64))
    assert np.all(np.abs(h_gpu - h_ref) <= H_REL * np.abs(h_ref) + 3e-37 * np.maximum(u_abs, 1.0))
    r_qs, r_d, r_s = oracle.quantize_act(h_gpu)
    assert np.array_equal(hq_qs, r_qs) and np.array_equal(hq_d, r_d) and np.array_equal(hq_s, r_s)

    say(f"FFN chain T={t}: down")
    ws_d = torch.zeros(qmv.moe_workspace_bytes(fmt, E_C4, K_C4, NFF_C4, t, TOPK_C4), dtype=torch.uint8,
                       device="cuda")
    y = qmv.moe_matvec(fmt, dn_w, E_C4, K_C4, NFF_C4, hq, True, ids_d, rw_d, ws_d).cpu().numpy()
    rw_h = rw_d.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(48), np.arange(K_C4 - 48, K_C4),
                                     synth.randint(synth.stream(f"ffn_c4/rows/{t}"), 0, 96, 0, K_C4 - 1)]))
    rb = dn_w.shape[1]
    v = dn_w.view(E_C4, K_C4, rb)
    dn_rows = v.index_select(0, torch.tensor(used, dtype=torch.int64, device="cuda")).index_select(
        1, torch.from_numpy(rows.astype(np.int64)).cuda()).contiguous().cpu().numpy()
    yr, mag = oracle.moe_matvec(fmt, dn_rows, len(used), len(rows), NFF_C4, r_qs, r_d, r_s, remap, rw_h, True)
    assert_y(y[:, rows], yr, mag, f"down T={t}")


@pytest.mark.parametrize("fmt,k", [(synth.Q8_0, 1056), (synth.Q4_K, 2048), (synth.IQ4_XS, 4096)],
                         ids=["q8_0_k1056", "q4_K_k2048", "iq4_xs_k4096"])
def test_gate_up_swiglu_fused(fmt, k):
    """qmv_moe_gate_up_swiglu's one-launch path (a workgroup holding a block's
    32 gate and 32 up rows makes that block of h in LDS) against its
    two-launch path, bit for bit, and against the oracle: one and two weight
    units per lane (the row lengths), duplicate experts inside a token and
    across tokens, dropped slots, calls in a row on one workspace, with and
    without the gate+up output."""
    qmv = need_gpu()
    e_n, n_ff, top_k = 6, 96, 4
    w = synth.make_weights(fmt, e_n * 2 * n_ff, k, f"fgu/{fmt}/{k}").data
    wd = to_dev(w)
    ws = torch.zeros(qmv.moe_workspace_bytes(fmt, e_n, 2 * n_ff, k, 16, top_k), dtype=torch.uint8, device="cuda")
    try:
        for t in (16, 6, 5, 1):
            ids, _ = synth.make_routing(t, e_n, top_k, f"fgu/r/{t}")
            ids = ids.copy()
            if t > 1:
                ids[0, 1] = ids[0, 0]  # a duplicate inside a token
                ids[t - 1, 2] = -1     # dropped slots
                ids[t // 2, 3] = e_n
            x = x_host(t, k, f"fgu/x/{fmt}/{t}")
            xq = quantize(qmv, x)
            ids_d = to_dev(ids)
            say(f"gate_up_swiglu fused {fmt} K={k} T={t}")
            qmv.set_tuning("ffn_fuse", 1)
            gu = torch.empty((t, top_k, 2 * n_ff), dtype=torch.float32, device="cuda")
            hq = qmv.moe_gate_up_swiglu(fmt, wd, e_n, n_ff, k, xq, ids_d, ws, gu=gu)
            hq_nogu = qmv.moe_gate_up_swiglu(fmt, wd, e_n, n_ff, k, xq, ids_d, ws)
            qmv.set_tuning("ffn_fuse", 0)
            gu2 = torch.empty_like(gu)
            hq2 = qmv.moe_gate_up_swiglu(fmt, wd, e_n, n_ff, k, xq, ids_d, ws, gu=gu2)
            assert torch.equal(gu, gu2), f"T={t}: gate+up sums differ between the paths"
            assert _same_q8(qmv, hq, hq2, t * top_k, n_ff), f"T={t}: Q8(h) differs between the paths"
            assert _same_q8(qmv, hq_nogu, hq2, t * top_k, n_ff), f"T={t}: Q8(h) without gu differs"
            qs, d, s = oracle.quantize_act(x)
            yr, mag = oracle.moe_matvec(fmt, w, e_n, 2 * n_ff, k, qs, d, s, ids, None, False)
            gu_h = gu.cpu().numpy()
            assert_y(gu_h, yr, mag, f"gate+up T={t}")
            h_gpu = torch.empty((t * top_k, n_ff), dtype=torch.float32, device="cuda")
            qmv.swiglu_quantize(gu.view(t * top_k, 2 * n_ff), n_ff, h_out=h_gpu)
            r_qs, r_d, r_s = oracle.quantize_act(h_gpu.cpu().numpy())
            h_qs, h_d, h_s = (a_.cpu().numpy() for a_ in qmv.act_fields(hq, t * top_k, n_ff))
            assert np.array_equal(h_qs, r_qs) and np.array_equal(h_d, r_d) and np.array_equal(h_s, r_s)
            drop = (ids < 0) | (ids >= e_n)
            assert np.all(h_qs.reshape(t, top_k, n_ff)[drop] == 0) and np.all(h_d.reshape(t, top_k, -1)[drop] == 0)
    finally:
        qmv.set_tuning("ffn_fuse", -1)
