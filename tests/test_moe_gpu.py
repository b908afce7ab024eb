"""qmv_moe_matvec (expert-grouped routed matvec) against the oracle.

The MoE decode workload: 128 IQ4_XS experts, gate+up 3072 x 4096 and down
4096 x 1536 per expert, top-8 routing, 1 / 6 / 16 / 64 tokens, on sampled
rows; plus routing edge cases on small expert sets (duplicate ids in one
token, one expert taking every slot, dropped ids, every id dropped)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y, gpu, need_gpu, quantize, sample_rows, say, to_dev, weights, x_host

pytestmark = gpu

E, TOP_K = 128, 8
GU = (3072, 4096)
DN = (4096, 1536)
NAME = "moe_iq4_xs_e128"


@pytest.fixture(scope="module")
def experts():
    need_gpu()
    say("MoE: generating expert weights")
    gu = weights(synth.IQ4_XS, E * GU[0], GU[1], f"{NAME}/gate_up")
    dn = weights(synth.IQ4_XS, E * DN[0], DN[1], f"{NAME}/down")
    return gu, dn


def _rows_of_experts(w_dev, n_rows, rows):
    """Host copy [E][len(rows)][row_bytes] of the chosen rows of every expert."""
    rb = w_dev.shape[1]
    v = w_dev.view(E, n_rows, rb)
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    return v.index_select(1, idx).contiguous().cpu().numpy()


@pytest.fixture(params=[1, 2, 3], ids=["vector", "matrix", "flat"])
def moe_kernel(request):
    """Run a test with the vector-ALU, the matrix-core and the few-slot flat
    MoE kernel."""
    qmv = need_gpu()
    qmv.set_tuning("moe_kernel", request.param)
    yield request.param
    qmv.set_tuning("moe_kernel", 0)


def _ws(qmv, n_rows, k, t):
    return torch.zeros(qmv.moe_workspace_bytes(synth.IQ4_XS, E, n_rows, k, t, TOP_K),
                       dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("t", [1, 6, 10, 16, 20, 64])
def test_moe_workload(experts, t, moe_kernel):
    qmv = need_gpu()
    gu, dn = experts
    ids, rw = synth.make_routing(t, E, TOP_K, f"{NAME}/route")
    ids_d, rw_d = to_dev(ids), to_dev(rw)

    # gate+up: x per token, one output per slot
    say(f"MoE gate_up T={t} kernel={moe_kernel}")
    n, k = GU
    x = x_host(t, k, f"{NAME}/x")
    xq = quantize(qmv, x)
    y = qmv.moe_matvec(synth.IQ4_XS, gu, E, n, k, xq, False, ids_d, None, _ws(qmv, n, k, t))
    rows = sample_rows(n, 96, f"{NAME}/gu_rows/{t}")
    w_h = _rows_of_experts(gu, n, rows)
    qs, d, s = oracle.quantize_act(x)
    yr, mag = oracle.moe_matvec(synth.IQ4_XS, w_h, E, len(rows), k, qs, d, s, ids, None, False)
    assert_y(y.cpu().numpy()[:, :, rows], yr, mag, f"gate_up T={t}")

    # down: x per slot, route-weighted sum over slots
    say(f"MoE down T={t}")
    n, k = DN
    h = x_host(t * TOP_K, k, f"{NAME}/h")
    hq = quantize(qmv, h)
    ws = _ws(qmv, n, k, t)
    for rep in range(2):  # the second call finds the counters reset
        y = qmv.moe_matvec(synth.IQ4_XS, dn, E, n, k, hq, True, ids_d, rw_d, ws)
        rows = sample_rows(n, 96, f"{NAME}/dn_rows/{t}")
        w_h = _rows_of_experts(dn, n, rows)
        qs, d, s = oracle.quantize_act(h)
        yr, mag = oracle.moe_matvec(synth.IQ4_XS, w_h, E, len(rows), k, qs, d, s, ids, rw, True)
        assert_y(y.cpu().numpy()[:, rows], yr, mag, f"down T={t} rep={rep}")
    assert int(ws[:4].view(torch.int32)[0]) == 0  # no dropped slots


SMALL_E, SMALL_N, SMALL_K = 6, 40, 512


@pytest.fixture(scope="module")
def small():
    need_gpu()
    w = synth.make_weights(synth.IQ4_XS, SMALL_E * SMALL_N, SMALL_K, "moe_small/w").data
    return w, to_dev(w)


CASES = {
    "duplicates": np.array([[0, 4, 4], [5, 5, 5], [2, 1, 2]], np.int32),
    "one_hot_expert": np.full((5, 3), 3, np.int32),
    "dropped": np.array([[0, -1, 2], [6, 1, 1000], [3, 3, -7]], np.int32),
    "all_dropped": np.array([[-1, 6], [7, -2]], np.int32),
    "single_token": np.array([[5, 0, 1, 2]], np.int32),
    "single_token_dropped": np.array([[5, -1, 1000, 2, 5]], np.int32),  # and a duplicate
    "single_token_all_dropped": np.array([[-1, 1000]], np.int32),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("per_slot", [False, True])
@pytest.mark.parametrize("weighted", [False, True])
def test_moe_routing_edges(small, case, per_slot, weighted, moe_kernel):
    qmv = need_gpu()
    w, wd = small
    ids = CASES[case]
    t, top_k = ids.shape
    say(f"MoE edge {case} per_slot={per_slot} weighted={weighted} kernel={moe_kernel}")
    rw = None
    if weighted:
        rw = synth.normal_f32(synth.stream(f"moe_small/rw/{case}"), 0, t * top_k).reshape(t, top_k)
    x = x_host(t * top_k if per_slot else t, SMALL_K, f"moe_small/x/{per_slot}")
    xq = quantize(qmv, x)
    ws = torch.zeros(qmv.moe_workspace_bytes(synth.IQ4_XS, SMALL_E, SMALL_N, SMALL_K, t, top_k),
                     dtype=torch.uint8, device="cuda")
    fill = torch.full((t * (1 if weighted else top_k) * SMALL_N,), 123.0, device="cuda")
    y = qmv.moe_matvec(synth.IQ4_XS, wd, SMALL_E, SMALL_N, SMALL_K, xq, per_slot, to_dev(ids),
                       None if rw is None else to_dev(rw), ws, y=fill)
    qs, d, s = oracle.quantize_act(x)
    yr, mag = oracle.moe_matvec(synth.IQ4_XS, w, SMALL_E, SMALL_N, SMALL_K, qs, d, s, ids, rw,
                                per_slot)
    assert_y(y.cpu().numpy().reshape(yr.shape), yr, mag, case)
    dropped = int(((ids < 0) | (ids >= SMALL_E)).sum())
    assert int(ws[:4].view(torch.int32)[0]) == dropped


def test_moe_matches_dense_calls(small):
    """T = 1: the routed call equals top_k dense matvecs of the chosen experts."""
    qmv = need_gpu()
    w, wd = small
    ids = np.array([[4, 1, 3]], np.int32)
    x = x_host(1, SMALL_K, "moe_small/dense")
    xq = quantize(qmv, x)
    ws = torch.zeros(qmv.moe_workspace_bytes(synth.IQ4_XS, SMALL_E, SMALL_N, SMALL_K, 1, 3),
                     dtype=torch.uint8, device="cuda")
    y = qmv.moe_matvec(synth.IQ4_XS, wd, SMALL_E, SMALL_N, SMALL_K, xq, False, to_dev(ids), None,
                       ws).cpu().numpy()
    rb = qmv.row_bytes(synth.IQ4_XS, SMALL_K)
    for s_, e in enumerate(ids[0]):
        sub = wd.view(-1)[int(e) * SMALL_N * rb:(int(e) + 1) * SMALL_N * rb]
        yd = qmv.matvec(synth.IQ4_XS, sub, SMALL_N, SMALL_K, xq, 1).cpu().numpy()
        qs, d, s = oracle.quantize_act(x)
        yr, mag = oracle.matvec(synth.IQ4_XS, w[int(e) * SMALL_N:(int(e) + 1) * SMALL_N], SMALL_K,
                                qs, d, s)
        assert_y(y[0, s_][None], yr, mag, f"slot {s_}")
        assert_y(yd, yr, mag, f"dense {e}")


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_K], ids=["q8_0", "q4_K"])
def test_moe_other_formats(fmt, moe_kernel):
    """Both MoE kernels on Q8_0 and q4_K experts (K = 512, a hot expert that
    takes more slots than one staged group, weighted and per-slot calls)."""
    qmv = need_gpu()
    e_n, n, k = 5, 48, 512
    w = synth.make_weights(fmt, e_n * n, k, f"moe_fmt/{fmt}").data
    wd = to_dev(w)
    ids = np.array([[1, 3], [3, 0], [3, 4], [2, 3], [3, 1], [0, 3], [3, 2], [4, 3], [3, 0], [1, 3],
                    [3, 4], [2, 3], [3, 1], [0, 3], [3, 2], [4, 3], [3, 4], [1, 3]], np.int32)
    t, top_k = ids.shape
    rw = synth.normal_f32(synth.stream(f"moe_fmt/rw/{fmt}"), 0, t * top_k).reshape(t, top_k)
    for per_slot, weighted in ((False, False), (True, True)):
        say(f"MoE fmt {fmt} per_slot={per_slot} weighted={weighted} kernel={moe_kernel}")
        x = x_host(t * top_k if per_slot else t, k, f"moe_fmt/x/{per_slot}")
        xq = quantize(qmv, x)
        ws = torch.zeros(qmv.moe_workspace_bytes(fmt, e_n, n, k, t, top_k), dtype=torch.uint8,
                         device="cuda")
        y = qmv.moe_matvec(fmt, wd, e_n, n, k, xq, per_slot, to_dev(ids),
                           to_dev(rw) if weighted else None, ws)
        qs, d, s = oracle.quantize_act(x)
        yr, mag = oracle.moe_matvec(fmt, w, e_n, n, k, qs, d, s, ids, rw if weighted else None,
                                    per_slot)
        assert_y(y.cpu().numpy().reshape(yr.shape), yr, mag, f"fmt {fmt} per_slot={per_slot}")


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_K, synth.IQ4_XS], ids=["q8_0", "q4_K", "iq4_xs"])
@pytest.mark.parametrize("kernel,row16", [(0, 0), (3, 1), (3, 0)], ids=["auto", "flat-row-per-wave", "flat-16-lane"])
def test_moe_one_token_weighted(fmt, kernel, row16):
    """One token with route weights: the few-slot kernels with the combine
    folded in (top_k <= 8) -- one row per wave (rows of up to two units per
    lane) and 16-lane row groups (rows of up to 64 blocks) -- on every MoE
    format, for rows of 16 to 128 blocks (K = 512 .. 4096; Q8_0 also 33
    blocks, a ragged last lane group), a row count that leaves the last
    workgroup's rows partly empty, one activation row per token and per slot,
    top_k 1 and 8, with a dropped id and a duplicate."""
    qmv = need_gpu()
    e_n, n = 9, 70
    qmv.set_tuning("moe_kernel", kernel)
    qmv.set_tuning("moe_row16", row16)
    ks = (512, 1056, 1536, 2048, 4096) if fmt == synth.Q8_0 else (512, 1536, 2048, 4096)
    try:
        for k in ks:
            w = synth.make_weights(fmt, e_n * n, k, f"moe1/{fmt}/{k}").data
            wd = to_dev(w)
            for ids in (np.array([[4]], np.int32), np.array([[7]], np.int32),
                        np.array([[2, 8, 0, 5, 1, 6, 3, 4]], np.int32),
                        np.array([[2, -1, 0, 5, 5, 6, 1000, 4]], np.int32)):
                top_k = ids.shape[1]
                rw = synth.normal_f32(synth.stream(f"moe1/rw/{top_k}"), 0, top_k).reshape(1, top_k)
                for per_slot in (False, True):
                    say(f"MoE one token {fmt} K={k} ids={ids.tolist()} per_slot={per_slot} kernel={kernel}")
                    x = x_host(top_k if per_slot else 1, k, f"moe1/x/{k}/{per_slot}")
                    xq = quantize(qmv, x)
                    ws = torch.zeros(qmv.moe_workspace_bytes(fmt, e_n, n, k, 1, top_k), dtype=torch.uint8,
                                     device="cuda")
                    y = qmv.moe_matvec(fmt, wd, e_n, n, k, xq, per_slot, to_dev(ids), to_dev(rw), ws)
                    qs, d, s = oracle.quantize_act(x)
                    yr, mag = oracle.moe_matvec(fmt, w, e_n, n, k, qs, d, s, ids, rw, per_slot)
                    assert_y(y.cpu().numpy().reshape(yr.shape), yr, mag, f"{fmt} K={k} top_k={top_k}")
                    dropped = int(((ids < 0) | (ids >= e_n)).sum())
                    assert int(ws[:4].view(torch.int32)[0]) == dropped
    finally:
        qmv.set_tuning("moe_kernel", 0)
        qmv.set_tuning("moe_row16", 0)
