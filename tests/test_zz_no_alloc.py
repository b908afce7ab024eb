"""qmv_moe_matvec_noalloc (the MoE routed matvec on the library's own
device-resident workspace) against qmv_moe_matvec with a caller workspace and
against the oracle: bit-identical to the workspace call (same kernels, same
order of operations) and within 1e-4 of the sum of |terms| of the oracle.
Two calls in a row, the second smaller than the first, so that what the first
left in the shared array cannot leak into the second."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y, gpu, need_gpu, quantize, say, to_dev, weights, x_host

pytestmark = gpu

E, TOP_K = 128, 8
DN = (4096, 1536)


def _case(qmv, fmt, wd, w_host_rows, e, n, k, t, top_k, weighted, per_slot, name):
    ids, rw = synth.make_routing(t, e, top_k, f"noalloc/{name}/route")
    ids = ids.copy()
    if t > 2:
        ids[1, 2] = -1  # a dropped slot
    x = x_host(t * top_k if per_slot else t, k, f"noalloc/{name}/x")
    xq = quantize(qmv, x)
    ids_d = to_dev(ids)
    rw_d = to_dev(rw) if weighted else None
    shape = (t, n) if weighted else (t, top_k, n)
    y0 = torch.full(shape, 7.0, dtype=torch.float32, device="cuda")
    y1 = torch.full(shape, -3.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(qmv.moe_workspace_bytes(fmt, e, n, k, t, top_k), dtype=torch.uint8, device="cuda")
    qmv.moe_matvec(fmt, wd, e, n, k, xq, per_slot, ids_d, rw_d, ws, y=y0)
    qmv.moe_matvec_noalloc(fmt, wd, e, n, k, xq, per_slot, ids_d, rw_d, y1)
    torch.cuda.synchronize()
    a, b = y0.cpu().numpy(), y1.cpu().numpy()
    assert np.array_equal(a, b), f"{name}: no-alloc call differs from the workspace call"
    qs, d, s = oracle.quantize_act(x)
    rows = w_host_rows[1]
    yr, mag = oracle.moe_matvec(fmt, w_host_rows[0], e, len(rows), k, qs, d, s, ids, rw if weighted else None,
                                per_slot)
    got = b[..., rows]
    assert_y(got, yr, mag, name)


def _rows_of_experts(w_dev, e, n, rows):
    rb = w_dev.shape[1]
    v = w_dev.view(e, n, rb)
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    return v.index_select(1, idx).contiguous().cpu().numpy()


def test_noalloc_matches_workspace_call_twice():
    qmv = need_gpu()
    fmt = synth.IQ4_XS
    n, k = DN
    say("no-alloc MoE: generating expert weights")
    wd = weights(fmt, E * n, k, "noalloc/down")
    rows = np.unique(np.concatenate([np.arange(40), np.arange(n - 40, n),
                                     synth.randint(synth.stream("noalloc/rows"), 0, 64, 0, n - 1)]))
    w_rows = (_rows_of_experts(wd, E, n, rows), rows)
    # first call: 64 tokens, route-weighted, one activation row per slot
    # (the largest per-slot output area of this workload); then a smaller one
    say("no-alloc MoE: 64 tokens weighted, per slot")
    _case(qmv, fmt, wd, w_rows, E, n, k, 64, TOP_K, True, True, "big")
    say("no-alloc MoE: 3 tokens weighted, per slot")
    _case(qmv, fmt, wd, w_rows, E, n, k, 3, TOP_K, True, True, "small")
    say("no-alloc MoE: 1 token weighted")
    _case(qmv, fmt, wd, w_rows, E, n, k, 1, TOP_K, True, True, "one")
    say("no-alloc MoE: 16 tokens, one output row per slot")
    _case(qmv, fmt, wd, w_rows, E, n, k, 16, TOP_K, False, True, "unweighted")


def test_noalloc_small_experts_other_formats():
    qmv = need_gpu()
    e, n, k, top_k = 6, 40, 512, 3
    for fmt in (synth.Q8_0, synth.Q4_K):
        w = synth.make_weights(fmt, e * n, k, f"noalloc/small/{fmt}").data
        wd = to_dev(w)
        rows = np.arange(n)
        for t, weighted in ((9, True), (2, False), (5, True)):
            say(f"no-alloc MoE small fmt={fmt} T={t} weighted={weighted}")
            _case(qmv, fmt, wd, (w, rows), e, n, k, t, top_k, weighted, False, f"small{fmt}/{t}")
