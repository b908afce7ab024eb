"""Split-K path of qmv_matvec (few rows, long K) against the oracle, forced
on and off, over repeated calls that must find the workspace counters reset."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y, gpu, host_rows, need_gpu, quantize, say, to_dev, weights, x_host

pytestmark = gpu


def _ref(fmt, w, k, x):
    qs, d, s = oracle.quantize_act(x)
    return oracle.matvec(fmt, w, k, qs, d, s)


def test_splitk_workload_256x65536():
    """The few-row long-K workload (Q8_0 256 x 65536, one token)."""
    qmv = need_gpu()
    name, fmt, n, k = "q8_0_splitk_256x65536", synth.Q8_0, 256, 65536
    wd = weights(fmt, n, k, f"{name}/W")
    w = wd.cpu().numpy()
    x = x_host(1, k, f"{name}/x")
    yr, mag = _ref(fmt, w, k, x)
    xq = quantize(qmv, x)
    ws = torch.zeros(qmv.matvec_workspace_bytes(fmt, n, k, 1), dtype=torch.uint8, device="cuda")
    try:
        for forced in (-1, 0, 2, 7, 16, 32, -1, 3):
            qmv.set_tuning("splitk", forced)
            for rep in range(3):
                say(f"split-K {name} slices={forced} rep={rep}")
                y = qmv.matvec(fmt, wd, n, k, xq, 1, ws=ws).cpu().numpy()
                assert_y(y, yr, mag, f"splitk={forced} rep={rep}")
        # no workspace: the single-pass kernel
        qmv.set_tuning("splitk", -1)
        y = qmv.matvec(fmt, wd, n, k, xq, 1).cpu().numpy()
        assert_y(y, yr, mag, "no workspace")
    finally:
        qmv.set_tuning("splitk", -1)
    # counters are back at zero after completed calls
    torch.cuda.synchronize()
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_K, synth.IQ4_XS, synth.Q5_K, synth.Q6_K, synth.Q8G128])
def test_splitk_all_formats_and_token_counts(fmt):
    qmv = need_gpu()
    n, k = 77, 8192
    w = synth.make_weights(fmt, n, k, f"sk/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"skx/{fmt}")
    try:
        for t in (1, 2, 5, 16):
            xq = quantize(qmv, x[:t])
            yr, mag = _ref(fmt, w, k, x[:t])
            ws = torch.zeros(qmv.matvec_workspace_bytes(fmt, n, k, t), dtype=torch.uint8,
                             device="cuda")
            for forced in (-1, 4, 9):
                qmv.set_tuning("splitk", forced)
                for rep in range(2):
                    say(f"split-K fmt={fmt} T={t} slices={forced} rep={rep}")
                    y = qmv.matvec(fmt, wd, n, k, xq, t, ws=ws).cpu().numpy()
                    assert_y(y, yr, mag, f"fmt {fmt} T={t} split {forced}")
    finally:
        qmv.set_tuning("splitk", -1)


def test_splitk_shares_workspace_across_shapes():
    """One workspace, sized for the larger call, serves a smaller one next."""
    qmv = need_gpu()
    fmt = synth.IQ4_XS
    big = qmv.matvec_workspace_bytes(fmt, 512, 16384, 4)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    try:
        qmv.set_tuning("splitk", 8)
        for n, k, t in ((512, 16384, 4), (40, 4096, 2), (512, 16384, 4)):
            w = synth.make_weights(fmt, n, k, f"sws/{n}").data
            x = x_host(t, k, f"swsx/{k}")
            y = qmv.matvec(fmt, to_dev(w), n, k, quantize(qmv, x), t, ws=ws).cpu().numpy()
            yr, mag = _ref(fmt, w, k, x)
            assert_y(y, yr, mag, f"shared ws N={n} K={k}")
    finally:
        qmv.set_tuning("splitk", -1)


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_K, synth.IQ4_XS, synth.Q8G128])
def test_matrix_core_split_over_workgroups(fmt):
    """The matrix-core kernel with K split over workgroups (a workspace and
    rows longer than one LDS chunk): every matrix-core variant, token counts
    of the three tile sizes, a ragged last row tile, repeated calls that must
    find the counters re-armed and give the same bits, and the unsplit kernel
    (no workspace) within the same tolerance."""
    qmv = need_gpu()
    n, k = 300, 14336
    w = synth.make_weights(fmt, n, k, f"mxs/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"mxsx/{fmt}")
    ws = torch.zeros(qmv.matvec_workspace_bytes(fmt, n, k, 16), dtype=torch.uint8, device="cuda")
    mx = [v for v in range(len(qmv.variants())) if qmv.variant_name(v).startswith("mx_")]
    assert mx
    try:
        for v in mx:
            qmv.set_tuning("variant", v)
            for t in (16, 9, 5, 3, 1):
                say(f"matrix-core split fmt={fmt} {qmv.variant_name(v)} T={t}")
                xq = quantize(qmv, x[:t])
                yr, mag = _ref(fmt, w, k, x[:t])
                first = None
                for rep in range(2):
                    y = qmv.matvec(fmt, wd, n, k, xq, t, ws=ws)
                    assert_y(y.cpu().numpy(), yr, mag, f"{qmv.variant_name(v)} T={t} rep={rep}")
                    if first is None:
                        first = y.clone()
                    else:
                        assert torch.equal(y, first), f"{qmv.variant_name(v)} T={t}"
                y0 = qmv.matvec(fmt, wd, n, k, xq, t).cpu().numpy()
                assert_y(y0, yr, mag, f"{qmv.variant_name(v)} T={t} unsplit")
    finally:
        qmv.set_tuning("variant", -1)
    torch.cuda.synchronize()
    assert int(ws[:2048 * 4].view(torch.int32).abs().sum()) == 0  # counters re-armed


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_K, synth.IQ4_XS, synth.Q5_K, synth.Q6_K, synth.Q8G128])
def test_flat_split_over_workgroups(fmt):
    """The LDS-staged flat kernel with K split over workgroups (a workspace,
    and rows longer than one chunk or too few rows to give every compute unit
    a workgroup): every such variant forced, 1/3/8 tokens, a ragged row count,
    repeated calls that must give the same bits and re-arm the counters."""
    qmv = need_gpu()
    n, k = 77, 8192
    w = synth.make_weights(fmt, n, k, f"fls/{fmt}").data
    wd = to_dev(w)
    x = x_host(8, k, f"flsx/{fmt}")
    ws = torch.zeros(qmv.matvec_workspace_bytes(fmt, n, k, 8), dtype=torch.uint8, device="cuda")
    staged = [v for v in range(len(qmv.variants()))
              if qmv.variant_name(v).startswith("fl_") and qmv.variant_name(v).endswith("_l")]
    assert staged
    split_seen = 0
    qmv.set_tuning("flat_split", 1)
    try:
        for v in staged:
            qmv.set_tuning("variant", v)
            for t in (1, 3, 8):
                split_seen += qmv.matvec_plan(fmt, n, k, t, True)[1] > 1
                say(f"flat split fmt={fmt} {qmv.variant_name(v)} T={t}")
                xq = quantize(qmv, x[:t])
                yr, mag = _ref(fmt, w, k, x[:t])
                first = None
                for rep in range(2):
                    y = qmv.matvec(fmt, wd, n, k, xq, t, ws=ws)
                    assert_y(y.cpu().numpy(), yr, mag, f"{qmv.variant_name(v)} T={t} rep={rep}")
                    if first is None:
                        first = y.clone()
                    else:
                        assert torch.equal(y, first), f"{qmv.variant_name(v)} T={t}"
    finally:
        qmv.set_tuning("variant", -1)
        qmv.set_tuning("flat_split", 0)
    assert split_seen > 0
    torch.cuda.synchronize()
    assert int(ws[:2048 * 4].view(torch.int32).abs().sum()) == 0  # counters re-armed


def test_flat_split_workload_256x65536():
    """The few-row long-K workload through every LDS-staged flat variant
    split over workgroups, one token, sampled against the oracle in full."""
    qmv = need_gpu()
    name, fmt, n, k = "q8_0_splitk_256x65536", synth.Q8_0, 256, 65536
    wd = weights(fmt, n, k, f"{name}/W")
    w = wd.cpu().numpy()
    x = x_host(1, k, f"{name}/x")
    yr, mag = _ref(fmt, w, k, x)
    xq = quantize(qmv, x)
    ws = torch.zeros(qmv.matvec_workspace_bytes(fmt, n, k, 1), dtype=torch.uint8, device="cuda")
    staged = [v for v in range(len(qmv.variants()))
              if qmv.variant_name(v).startswith("fl_") and qmv.variant_name(v).endswith("_l")]
    qmv.set_tuning("flat_split", 1)
    try:
        for v in staged:
            qmv.set_tuning("variant", v)
            assert qmv.matvec_plan(fmt, n, k, 1, True)[1] > 1
            say(f"flat split {name} {qmv.variant_name(v)}")
            y = qmv.matvec(fmt, wd, n, k, xq, 1, ws=ws).cpu().numpy()
            assert_y(y, yr, mag, qmv.variant_name(v))
    finally:
        qmv.set_tuning("variant", -1)
        qmv.set_tuning("flat_split", 0)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.IQ4_XS])
def test_matrix_core_forced_slice_counts(fmt):
    """Forced K slice counts of the matrix-core split (tuning key mx_slices),
    including counts whose slices would not fit and so take more, on a
    single-chunk and a multi-chunk row; 0 turns the split off."""
    qmv = need_gpu()
    v16 = qmv.variants().index("mx_w16_k4_r2")
    try:
        qmv.set_tuning("variant", v16)
        for n, k in ((96, 4096), (200, 14336)):
            w = synth.make_weights(fmt, n, k, f"mxf/{fmt}/{k}").data
            wd = to_dev(w)
            x = x_host(16, k, f"mxfx/{k}")
            ws = torch.zeros(qmv.matvec_workspace_bytes(fmt, n, k, 16), dtype=torch.uint8, device="cuda")
            for t in (16, 6):
                xq = quantize(qmv, x[:t])
                yr, mag = _ref(fmt, w, k, x[:t])
                for sl in (0, 2, 3, 5, 32, -1):
                    qmv.set_tuning("mx_slices", sl)
                    say(f"forced mx slices fmt={fmt} N={n} K={k} T={t} slices={sl}")
                    y = qmv.matvec(fmt, wd, n, k, xq, t, ws=ws).cpu().numpy()
                    assert_y(y, yr, mag, f"N={n} K={k} T={t} slices={sl}")
    finally:
        qmv.set_tuning("mx_slices", -1)
        qmv.set_tuning("variant", -1)
