"""qmv_matvec_x: the decode step from fp32 activations, with the matvec
workgroups quantizing x themselves where that is faster (Q8_0 at one or two
tokens, q4_K at one; every LDS-staged flat variant when forced).

  * xq bit-exact against the oracle's quantization of x, and the same bytes
    as qmv_quantize_act writes;
  * y bit-identical to qmv_matvec over qmv_quantize_act's buffer when both
    run the same kernel variant (every LDS-staged flat variant, forced), and
    within 1e-4 of the sum of |per-block terms| of the oracle with the
    automatic choice;
  * the two-launch path (three tokens and more) gives the same results;
  * edges: one block of K, one row, a row stride beyond K, zero blocks, long
    rows whose quantization takes more passes than the kernel holds in
    registers, and the full workload shapes on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y, gpu, host_rows, need_gpu, sample_rows, say, to_dev, weights, x_host

pytestmark = gpu

FMTS = [synth.Q8_0, synth.Q4_K, synth.IQ4_XS, synth.Q5_K, synth.Q6_K, synth.Q8G128]
NAMES = {synth.Q8_0: "q8_0", synth.Q4_K: "q4_K", synth.IQ4_XS: "iq4_xs", synth.Q5_K: "q5_K", synth.Q6_K: "q6_K",
         synth.Q8G128: "q8g128"}


def _check_xq(qmv, xq, x):
    t, k = x.shape
    qs, d, s = oracle.quantize_act(x)
    g_qs, g_d, g_s = (a.cpu().numpy() for a in qmv.act_fields(xq, t, k))
    assert np.array_equal(g_qs, qs) and np.array_equal(g_d, d) and np.array_equal(g_s, s)
    return qs, d, s


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_fused_equals_two_launches_every_staged_variant(fmt):
    qmv = need_gpu()
    n, k = 333, 2048
    w = synth.make_weights(fmt, n, k, f"fx/{fmt}").data
    wd = to_dev(w)
    x = x_host(2, k, f"fxx/{fmt}")
    staged = [i for i, nm in enumerate(qmv.variants()) if nm.startswith("fl_") and nm.endswith("_l")]
    assert staged
    try:
        for v in staged:
            qmv.set_tuning("variant", v)
            for t in (1, 2):
                say(f"matvec_x {NAMES[fmt]} {qmv.variant_name(v)} T={t}")
                xt = to_dev(x[:t])
                y, xq = qmv.matvec_x(fmt, wd, n, k, xt)
                ref = qmv.matvec(fmt, wd, n, k, qmv.quantize_act(xt), t)
                torch.cuda.synchronize()
                assert torch.equal(y, ref), f"{qmv.variant_name(v)} T={t}"
                qs, d, s = _check_xq(qmv, xq, x[:t])
                yr, mag = oracle.matvec(fmt, w, k, qs, d, s)
                assert_y(y.cpu().numpy(), yr, mag, f"{NAMES[fmt]} {qmv.variant_name(v)} T={t}")
    finally:
        qmv.set_tuning("variant", -1)


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_fused_automatic_and_two_launch_path(fmt):
    qmv = need_gpu()
    n, k = 300, 4096
    w = synth.make_weights(fmt, n, k, f"fa/{fmt}").data
    wd = to_dev(w)
    x = x_host(5, k, f"fax/{fmt}")
    for t in (1, 2, 3, 5):
        say(f"matvec_x auto {NAMES[fmt]} T={t}")
        y, xq = qmv.matvec_x(fmt, wd, n, k, to_dev(x[:t]))
        qs, d, s = _check_xq(qmv, xq, x[:t])
        yr, mag = oracle.matvec(fmt, w, k, qs, d, s)
        assert_y(y.cpu().numpy(), yr, mag, f"{NAMES[fmt]} T={t}")


def test_fused_edges():
    qmv = need_gpu()
    cases = [
        (synth.Q8_0, 1, 32, 1), (synth.Q8_0, 7, 32, 2),       # one block of K
        (synth.Q4_K, 1, 256, 2), (synth.IQ4_XS, 3, 256, 1),   # one super-block, one row
        (synth.Q4_K, 64, 14336, 2),                           # more quantization passes than registers hold
        (synth.IQ4_XS, 40, 14336, 2), (synth.Q6_K, 9, 768, 2),
        (synth.Q8G128, 5, 128, 2), (synth.Q8G128, 33, 5120, 1),   # 130-byte rows; the head's K
    ]
    for fmt, n, k, t in cases:
        say(f"matvec_x edge {NAMES[fmt]} N={n} K={k} T={t}")
        w = synth.make_weights(fmt, n, k, f"fe/{fmt}/{n}/{k}").data
        x = x_host(t, k, f"fex/{k}/{t}")
        x[0, 32:64] = 0.0  # a zero block
        # a row stride beyond K: x rows inside a wider buffer
        xb = torch.zeros((t, k + 64), dtype=torch.float32, device="cuda")
        xb[:, :k] = to_dev(x)
        y, xq = qmv.matvec_x(fmt, to_dev(w), n, k, xb[:, :k])
        qs, d, s = _check_xq(qmv, xq, x)
        yr, mag = oracle.matvec(fmt, w, k, qs, d, s)
        assert_y(y.cpu().numpy(), yr, mag, f"edge {NAMES[fmt]} N={n} K={k} T={t}")


FULL = [
    ("q4_k_14336x4096", synth.Q4_K, 14336, 4096),
    ("iq4_xs_4096x14336", synth.IQ4_XS, 4096, 14336),
    ("q8_0_4096x4096", synth.Q8_0, 4096, 4096),
    ("q8_0_head_152064x5120", synth.Q8_0, 152064, 5120),
]


@pytest.mark.parametrize("name,fmt,n,k", FULL, ids=[c[0] for c in FULL])
def test_fused_full_shapes(name, fmt, n, k):
    qmv = need_gpu()
    say(f"matvec_x full {name}: generating weights")
    wd = weights(fmt, n, k, f"{name}/W")
    rows = sample_rows(n, 256, f"frows/{name}")
    wh = host_rows(wd, rows)
    x = x_host(2, k, f"{name}/x")
    for t in (1, 2):
        say(f"matvec_x full {name} T={t}")
        y, xq = qmv.matvec_x(fmt, wd, n, k, to_dev(x[:t]))
        qs, d, s = _check_xq(qmv, xq, x[:t])
        yr, mag = oracle.matvec(fmt, wh, k, qs, d, s)
        assert_y(y.cpu().numpy()[:, rows], yr, mag, f"{name} T={t}")


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.IQ4_XS, synth.Q8_0])
def test_fused_with_workspace_matches_split_matvec(fmt):
    """With a split-K workspace the two-launch path runs the same split
    matvec as qmv_matvec with that workspace: the same bits, on a few-row
    long-K shape at every tile size."""
    qmv = need_gpu()
    n, k = 300, 14336
    w = synth.make_weights(fmt, n, k, f"fws/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"fwsx/{fmt}")
    ws = torch.zeros(qmv.matvec_workspace_bytes(fmt, n, k, 16), dtype=torch.uint8, device="cuda")
    for t in (1, 5, 16):
        say(f"matvec_x with workspace {NAMES[fmt]} T={t}")
        xt = to_dev(x[:t])
        y, xq = qmv.matvec_x(fmt, wd, n, k, xt, ws=ws)
        ref = qmv.matvec(fmt, wd, n, k, qmv.quantize_act(xt), t, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"T={t}"
        qs, d, s = _check_xq(qmv, xq, x[:t])
        yr, mag = oracle.matvec(fmt, w, k, qs, d, s)
        assert_y(y.cpu().numpy(), yr, mag, f"{NAMES[fmt]} T={t} ws")
