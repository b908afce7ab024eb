"""qmv_router_topk (router matvec, top-k, softmax over the chosen) against
the oracle.

The logits are fp32 sums on the GPU: each is compared with the oracle's fp64
logit within 1e-4 of the sum of |w_i x_i| (the matvec tolerance).  Which
experts are chosen is an integer decision taken from those fp32 logits, so the
ids must equal the oracle's selection from the GPU's own logits exactly (same
order rule: larger logit first, lower index on ties), and the weights the
oracle's softmax of those logits within 1e-6 relative.

With an activation buffer the router also writes the Q8 blocks of x: those
bytes must equal the oracle's quantization of x and qmv_quantize_act's output
exactly."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import gpu, need_gpu, say, to_dev

pytestmark = gpu


def _check(qmv, x: np.ndarray, wr: np.ndarray, top_k: int, what: str):
    t, e = x.shape[0], wr.shape[0]
    logits_d = torch.empty((t, e), dtype=torch.float32, device="cuda")
    ids_d, w_d = qmv.router_topk(to_dev(x), to_dev(wr), top_k, logits=logits_d)
    logits, ids, w = logits_d.cpu().numpy(), ids_d.cpu().numpy(), w_d.cpu().numpy()
    _, _, l_ref = oracle.router_topk(x, wr, top_k)
    mag = np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)).T
    err = np.abs(logits.astype(np.float64) - l_ref)
    assert np.all(err <= 1e-4 * mag), (what, float((err / np.maximum(mag, 1e-300)).max()))
    ids_ref, w_ref = oracle.topk_from_logits(logits, top_k)
    assert np.array_equal(ids, ids_ref), (what, ids[:2], ids_ref[:2])
    assert np.allclose(w, w_ref, rtol=1e-6, atol=1e-7), what
    assert np.allclose(w.sum(1), 1.0, atol=1e-5)
    return ids, w


@pytest.mark.parametrize("t", [1, 4, 16, 64])
def test_router_workload(t):
    """128 experts over K = 4096 (the MoE decode workload), top-8."""
    qmv = need_gpu()
    say(f"router T={t}")
    x = synth.make_x(t, 4096, "router/x")
    wr = synth.make_x(128, 4096, "router/w") * np.float32(0.02)
    _check(qmv, x, wr, 8, f"T={t}")


def test_router_ties_and_shapes():
    qmv = need_gpu()
    say("router ties")
    e, k = 200, 64
    wr = np.zeros((e, k), np.float32)
    for i in range(e):
        wr[i, i % k] = 1.0  # experts i and i + 64 share a logit
    x = np.zeros((3, k), np.float32)
    x[0] = np.arange(k, dtype=np.float32) % 7  # many exact ties
    x[1] = 1.0  # every logit tied
    x[2] = -np.arange(k, dtype=np.float32)
    ids, _ = _check(qmv, x, wr, 16, "ties")
    assert ids[1].tolist() == list(range(16))
    # top_k = n_experts, one expert, odd expert count
    _check(qmv, synth.make_x(2, 128, "router/x2"), synth.make_x(5, 128, "router/w2"), 5, "all")
    _check(qmv, synth.make_x(2, 128, "router/x3"), synth.make_x(1, 128, "router/w3"), 1, "one")
    ids, w = _check(qmv, synth.make_x(3, 1024, "router/x4"), synth.make_x(1024, 1024, "router/w4"), 16,
                    "1024 experts")
    assert len(set(ids[0].tolist())) == 16


def test_router_feeds_moe():
    """The router's ids and weights drive qmv_moe_matvec directly."""
    qmv = need_gpu()
    e_n, n, k, top_k, t = 6, 40, 512, 2, 3
    x = synth.make_x(t, k, "router_moe/x")
    wr = synth.make_x(e_n, k, "router_moe/wr")
    xq = torch.empty(qmv.act_bytes(t, k), dtype=torch.uint8, device="cuda")
    ids_d, w_d = qmv.router_topk(to_dev(x), to_dev(wr), top_k, xq=xq)
    w = synth.make_weights(synth.IQ4_XS, e_n * n, k, "router_moe/w").data
    ws = torch.zeros(qmv.moe_workspace_bytes(synth.IQ4_XS, e_n, n, k, t, top_k), dtype=torch.uint8,
                     device="cuda")
    y = qmv.moe_matvec(synth.IQ4_XS, to_dev(w), e_n, n, k, xq, False, ids_d, w_d, ws).cpu().numpy()
    qs, d, s = oracle.quantize_act(x)
    yr, mag = oracle.moe_matvec(synth.IQ4_XS, w, e_n, n, k, qs, d, s, ids_d.cpu().numpy(),
                                w_d.cpu().numpy(), False)
    assert np.all(np.abs(y - yr) <= 1e-4 * mag)


@pytest.mark.parametrize("t,k,e", [(1, 4096, 128), (2, 4096, 128), (3, 1056, 7), (4, 32, 3), (5, 96, 40),
                                   (16, 2048, 64), (64, 4096, 128), (1, 5120, 1)])
def test_router_writes_q8_of_x(t, k, e):
    """The optional Q8 output: every token, every block, with a zero block and
    a row stride beyond K; K spans the kernel's two-chunk loop and its tail."""
    qmv = need_gpu()
    say(f"router xq T={t} K={k} E={e}")
    x = synth.make_x(t, k, f"router_xq/{t}/{k}")
    x[0, :32] = 0.0
    wr = synth.make_x(e, k, f"router_xq/w/{e}/{k}")
    xb = torch.zeros((t, k + 64), dtype=torch.float32, device="cuda")
    xb[:, :k] = to_dev(x)
    xq = torch.full((qmv.act_bytes(t, k),), 0xA5, dtype=torch.uint8, device="cuda")
    logits_d = torch.empty((t, e), dtype=torch.float32, device="cuda")
    ids_d, _ = qmv.router_topk(xb[:, :k], to_dev(wr), min(2, e), logits=logits_d, xq=xq)
    ref = qmv.quantize_act(xb[:, :k])
    torch.cuda.synchronize()
    for got, want in zip(qmv.act_fields(xq, t, k), qmv.act_fields(ref, t, k)):
        assert torch.equal(got, want)
    qs, d, s = oracle.quantize_act(x)
    g_qs, g_d, g_s = (a.cpu().numpy() for a in qmv.act_fields(xq, t, k))
    assert np.array_equal(g_qs, qs) and np.array_equal(g_d, d) and np.array_equal(g_s, s)
    # the selection is unchanged by the extra output
    ids2, _ = qmv.router_topk(xb[:, :k], to_dev(wr), min(2, e))
    assert torch.equal(ids_d, ids2)
