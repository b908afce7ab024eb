"""Exact block integers of the matrix-core paths against the oracle.

qmv_block_dots_mx runs the matrix-core matvec kernel (activation staging,
weight loads, decode, zero-masked int8 matrix-core products) in its integer
mode; qmv_moe_block_dots does the same for the expert-grouped matrix-core
MoE kernel.  Every integer must equal oracle.block_dots bit for bit:

  * every matrix-core variant at every token count 1..16, on 333 rows (a
    ragged row tile) and, for Q8_0 and Q8G128, rows that end inside a
    super-block;
  * rows several LDS chunks long, and the K split over workgroups (forced
    slice counts and the automatic plan);
  * the full workload shapes (q4_K 14336 x 4096, IQ4_XS 4096 x 14336, the
    Q8_0 head's row slice) in the launch configuration qmv_matvec runs;
  * the MoE kernel with 4 and 8 staged slot rows, one activation row per
    token or per slot, duplicate and dropped ids, and the 128-expert gate+up
    shape at 16 tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import gpu, need_gpu, quantize, say, to_dev, weights, x_host

pytestmark = gpu

MX_FMTS = [synth.Q8_0, synth.Q4_K, synth.IQ4_XS, synth.Q8G128]
NAMES = {synth.Q8_0: "q8_0", synth.Q4_K: "q4_K", synth.IQ4_XS: "iq4_xs", synth.Q8G128: "q8g128"}


def _mx_variants(qmv):
    """The matrix-core variants: the persistent kernel (mx_) and the flat one (mf_)."""
    return [v for v in range(len(qmv.variants())) if qmv.variant_name(v).startswith(("mx_", "mf_"))]


def _ref(fmt, w, k, x):
    qs, _, s = oracle.quantize_act(x)
    return oracle.block_dots(fmt, w, k, qs, s)


def _first_diff(got, ref):
    i = tuple(int(v) for v in np.argwhere(got != ref)[0])
    return f"{int((got != ref).sum())} integers differ, first at {i}: gpu {got[i]} oracle {ref[i]}"


@pytest.mark.parametrize("fmt", MX_FMTS, ids=[NAMES[f] for f in MX_FMTS])
def test_every_variant_and_token_count(fmt):
    qmv = need_gpu()
    n = 333
    # Q8_0 / Q8G128 rows that end inside a super-block of eight 32-blocks
    k = {synth.Q8_0: 1056, synth.Q8G128: 1152}.get(fmt, 2048)
    w = synth.make_weights(fmt, n, k, f"mxd/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"mxdx/{fmt}")
    for t in range(1, 17):
        xq = quantize(qmv, x[:t])
        ref = _ref(fmt, w, k, x[:t])
        for v in _mx_variants(qmv):
            say(f"block_dots_mx {NAMES[fmt]} {qmv.variant_name(v)} N={n} K={k} T={t}")
            got = qmv.block_dots_mx(fmt, wd, n, k, xq, t, variant=v).cpu().numpy()
            assert np.array_equal(got, ref), f"{qmv.variant_name(v)} T={t}: {_first_diff(got, ref)}"


@pytest.mark.parametrize("fmt", MX_FMTS, ids=[NAMES[f] for f in MX_FMTS])
def test_long_rows_chunks_and_slices(fmt):
    """K = 14336 at 5, 9 and 16 tokens: several LDS chunks per row unsplit,
    and split over workgroups into 2, 3, 4 slices and the automatic plan."""
    qmv = need_gpu()
    n, k = 77, 14336
    w = synth.make_weights(fmt, n, k, f"mxl/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"mxlx/{fmt}")
    for t in (5, 9, 16):
        xq = quantize(qmv, x[:t])
        ref = _ref(fmt, w, k, x[:t])
        for v in _mx_variants(qmv):
            for slices in (0, -1, 2, 3, 4):
                say(f"block_dots_mx {NAMES[fmt]} {qmv.variant_name(v)} K={k} T={t} slices={slices}")
                try:
                    got = qmv.block_dots_mx(fmt, wd, n, k, xq, t, variant=v, slices=slices).cpu().numpy()
                except qmv.QmvError as e:
                    # that many slices do not fit; the flat kernel needs a slice
                    # that fits one workgroup's LDS
                    assert e.status == 2 and (slices >= 2 or qmv.variant_name(v).startswith("mf_")), str(e)
                    continue
                assert np.array_equal(got, ref), (f"{qmv.variant_name(v)} T={t} slices={slices}: "
                                                  f"{_first_diff(got, ref)}")


@pytest.mark.parametrize("fmt,n,k,tokens", [
    (synth.Q4_K, 14336, 4096, (2, 4, 8, 16)),
    (synth.IQ4_XS, 4096, 14336, (3, 4, 8, 16)),
    (synth.Q8_0, 4096, 4096, (9, 16)),
], ids=["q4_K_14336x4096", "iq4_xs_4096x14336", "q8_0_4096x4096"])
def test_workload_shapes(fmt, n, k, tokens):
    """The full workload shapes, every row, in qmv_matvec's own launch
    configuration with a workspace (variant and K split chosen as it
    chooses them)."""
    qmv = need_gpu()
    wd = weights(fmt, n, k, f"mxw/{fmt}")
    w = wd.cpu().numpy()
    x = x_host(16, k, f"mxwx/{fmt}")
    for t in tokens:
        say(f"block_dots_mx {NAMES[fmt]} {n}x{k} T={t} (qmv_matvec's plan)")
        xq = quantize(qmv, x[:t])
        got = qmv.block_dots_mx(fmt, wd, n, k, xq, t, variant=-1, slices=-1).cpu().numpy()
        ref = _ref(fmt, w, k, x[:t])
        assert np.array_equal(got, ref), f"T={t}: {_first_diff(got, ref)}"
        del got


def test_q8_0_head_slice():
    """Rows of the Q8_0 output head (K = 5120) at 16 tokens."""
    qmv = need_gpu()
    fmt, n, k = synth.Q8_0, 2048, 5120
    w = synth.make_weights(fmt, 152064, k, "mxh", rows=(70000, 70000 + n)).data
    wd = to_dev(w)
    x = x_host(16, k, "mxhx")
    xq = quantize(qmv, x)
    ref = _ref(fmt, w, k, x)
    for v in _mx_variants(qmv):
        say(f"block_dots_mx head slice {qmv.variant_name(v)}")
        got = qmv.block_dots_mx(fmt, wd, n, k, xq, 16, variant=v).cpu().numpy()
        assert np.array_equal(got, ref), f"{qmv.variant_name(v)}: {_first_diff(got, ref)}"


def _moe_ref(fmt, w, e, n, k, x, ids, per_slot):
    qs, _, s = oracle.quantize_act(x)
    t, top_k = ids.shape
    nc = 2 if fmt == synth.Q4_K else 1
    rb = oracle.row_bytes(fmt, k)
    w2 = w.reshape(e * n, rb)
    ref = np.zeros((t * top_k, n, k // 32, nc), np.int32)
    for ti in range(t):
        for si in range(top_k):
            ex = int(ids[ti, si])
            if not 0 <= ex < e:
                continue
            xr = ti * top_k + si if per_slot else ti
            ref[ti * top_k + si] = oracle.block_dots(fmt, w2[ex * n:(ex + 1) * n], k, qs[xr:xr + 1],
                                                     s[xr:xr + 1])[0]
    return ref


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_K, synth.IQ4_XS], ids=["q8_0", "q4_K", "iq4_xs"])
def test_moe_matrix_core_integers(fmt):
    qmv = need_gpu()
    e, n, top_k = 16, 200, 8
    k = 1536 if fmt != synth.Q8_0 else 1504
    w = synth.make_weights(fmt, e * n, k, f"mxm/{fmt}").data
    wd = to_dev(w)
    for t in (5, 16, 33, 64):
        ids, _ = synth.make_routing(t, e, top_k, f"mxm/r/{t}")
        ids = ids.copy()
        ids[0, 1] = ids[0, 0] if t > 1 else ids[0, 1]  # a duplicate expert in one token
        ids[t - 1, 3] = -1                             # dropped slots
        ids[t // 2, 5] = e
        for per_slot in (False, True):
            x = x_host(t * top_k if per_slot else t, k, f"mxm/x/{t}/{per_slot}")
            xq = quantize(qmv, x)
            ref = _moe_ref(fmt, w, e, n, k, x, ids, per_slot)
            ws = torch.zeros(qmv.moe_workspace_bytes(fmt, e, n, k, t, top_k), dtype=torch.uint8, device="cuda")
            for slot_rows in (4, 8):
                say(f"moe_block_dots {fmt} T={t} per_slot={per_slot} slot_rows={slot_rows}")
                got = qmv.moe_block_dots(fmt, wd, e, n, k, xq, per_slot, to_dev(ids), ws,
                                         slot_rows=slot_rows).cpu().numpy()
                assert np.array_equal(got, ref), f"T={t} slot_rows={slot_rows}: {_first_diff(got, ref)}"


def test_moe_gate_up_workload_16_tokens():
    """The 128-expert IQ4_XS gate+up shape (3072 x 4096 per expert) at 16
    tokens, the routing of the MoE workload, the automatic slot-row count."""
    qmv = need_gpu()
    fmt, e, n, k, t, top_k = synth.IQ4_XS, 128, 3072, 4096, 16, 8
    wd = weights(fmt, e * n, k, "mxg")
    ids, _ = synth.make_routing(t, e, top_k, "mxg/route")
    x = x_host(t, k, "mxg/x")
    xq = quantize(qmv, x)
    ws = torch.zeros(qmv.moe_workspace_bytes(fmt, e, n, k, t, top_k), dtype=torch.uint8, device="cuda")
    say("moe_block_dots gate+up 128x3072x4096 T=16")
    got = qmv.moe_block_dots(fmt, wd, e, n, k, xq, False, to_dev(ids), ws).cpu().numpy()
    used = sorted(set(ids.reshape(-1).tolist()))
    qs, _, s = oracle.quantize_act(x)
    for ex in used:
        w_e = wd[ex * n:(ex + 1) * n].cpu().numpy()
        ref_e = oracle.block_dots(fmt, w_e, k, qs, s)  # [T][n][nb][1]
        for ti in range(t):
            for si in range(top_k):
                if ids[ti, si] == ex:
                    g = got[ti * top_k + si]
                    assert np.array_equal(g, ref_e[ti]), f"expert {ex} slot {(ti, si)}: {_first_diff(g, ref_e[ti])}"
