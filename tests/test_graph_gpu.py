"""Calls captured in a HIP graph and replayed.  The library allocates
nothing, keeps no pointer after a call, and its split-K and MoE counters
re-arm inside the kernels (no memset node), so a captured sequence can be
replayed: every replay, with eager work and synchronisations between the
replays, must give the bits of the same calls run eagerly.

The sequence covers the paths with cross-workgroup state or fusion: the
matrix-core kernel split over workgroups (IQ4_XS, few rows, long K, 16
tokens, with a workspace), the fused decode step qmv_matvec_x (q4_K, one
token), the router writing the Q8 blocks of the MoE input, and the one-token
route-weighted MoE call (the flat kernel with the combine folded in) on them."""
import numpy as np
import torch

import synth
from gpu_util import gpu, need_gpu, say, to_dev, x_host

pytestmark = gpu


def test_graph_replays_match_eager():
    qmv = need_gpu()
    n1, k1, t1 = 300, 14336, 16
    w1 = to_dev(synth.make_weights(synth.IQ4_XS, n1, k1, "graph/w1").data)
    x1 = to_dev(x_host(t1, k1, "graph/x1"))
    ws1 = torch.zeros(qmv.matvec_workspace_bytes(synth.IQ4_XS, n1, k1, t1), dtype=torch.uint8, device="cuda")
    assert qmv.matvec_plan(synth.IQ4_XS, n1, k1, t1, True)[1] > 1  # the split path
    n2, k2 = 4096, 4096
    w2 = to_dev(synth.make_weights(synth.Q4_K, n2, k2, "graph/w2").data)
    x2 = to_dev(x_host(1, k2, "graph/x2"))
    n_exp, nr, kk, top_k = 16, 256, 1536, 4
    we = to_dev(synth.make_weights(synth.IQ4_XS, n_exp * nr, kk, "graph/we").data)
    ids = to_dev(np.array([[3, 7, 0, 12]], np.int32))
    rw = to_dev(np.array([[0.4, 0.3, 0.2, 0.1]], np.float32))
    xh = to_dev(x_host(top_k, kk, "graph/xh"))
    wrt = to_dev(x_host(n_exp, kk, "graph/wr"))
    wsm = torch.zeros(qmv.moe_workspace_bytes(synth.IQ4_XS, n_exp, nr, kk, 1, top_k), dtype=torch.uint8,
                      device="cuda")

    def buffers():
        return {
            "xq1": torch.empty(qmv.act_bytes(t1, k1), dtype=torch.uint8, device="cuda"),
            "y1": torch.empty((t1, n1), dtype=torch.float32, device="cuda"),
            "xq2": torch.empty(qmv.act_bytes(1, k2), dtype=torch.uint8, device="cuda"),
            "y2": torch.empty((1, n2), dtype=torch.float32, device="cuda"),
            "xqh": torch.empty(qmv.act_bytes(top_k, kk), dtype=torch.uint8, device="cuda"),
            "y3": torch.empty((1, nr), dtype=torch.float32, device="cuda"),
            "rid": torch.empty((top_k, top_k), dtype=torch.int32, device="cuda"),
            "rw": torch.empty((top_k, top_k), dtype=torch.float32, device="cuda"),
            "rl": torch.empty((top_k, n_exp), dtype=torch.float32, device="cuda"),
        }

    def step(o):
        qmv.quantize_act(x1, out=o["xq1"])
        qmv.matvec(synth.IQ4_XS, w1, n1, k1, o["xq1"], t1, y=o["y1"], ws=ws1)
        qmv.matvec_x(synth.Q4_K, w2, n2, k2, x2, xq=o["xq2"], y=o["y2"])
        qmv.router_topk(xh, wrt, top_k, ids=o["rid"], weights=o["rw"], logits=o["rl"], xq=o["xqh"])
        qmv.moe_matvec(synth.IQ4_XS, we, n_exp, nr, kk, o["xqh"], True, ids, rw, wsm, y=o["y3"])

    say("graph: eager reference")
    ref = buffers()
    step(ref)
    torch.cuda.synchronize()

    say("graph: capture")
    out = buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    other = buffers()
    for rep in range(4):
        say(f"graph: replay {rep}")
        for v in out.values():
            v.fill_(0)  # the replay must rewrite every output
        g.replay()
        torch.cuda.synchronize()
        for name in ("y1", "y2", "y3", "xq1", "xq2", "rid", "rw", "rl"):
            assert torch.equal(out[name], ref[name]), (rep, name)
        for got, want in zip(qmv.act_fields(out["xqh"], top_k, kk), qmv.act_fields(ref["xqh"], top_k, kk)):
            assert torch.equal(got, want), (rep, "xqh")
        step(other)  # eager work on the same weights and workspaces between replays
        torch.cuda.synchronize()
        for name in ("y1", "y2", "y3"):
            assert torch.equal(other[name], ref[name]), (rep, name, "eager")
    # the counters the replays used are back at zero
    assert int(ws1[:2048 * 4].view(torch.int32).abs().sum()) == 0
