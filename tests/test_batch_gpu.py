"""qmv_matvec_batch (sibling matvecs sharing one activation buffer in one
launch, each optionally plus a residual) against the oracle.

  * every kernel variant and a spread of token counts on small ragged
    siblings (row counts that leave every kind of padding between the
    matrices), residuals on some of them, one accumulating in place, output
    columns past n_rows left untouched;
  * a one-item batch equals qmv_matvec bit for bit, and with a residual the
    fp32 sum of qmv_matvec's output and the residual;
  * the full sibling shapes (q4_K gate and up 2 x 14336 x 4096, IQ4_XS
    2 x 4096 x 14336) at their token counts on sampled rows, in the launch
    configuration the bench times;
  * eight items (the maximum), one-row items, repeated in-place calls.
Rule: |y - y*| <= 1e-4 * (sum|terms| + |r|), the residual counted as one
more term of the sum.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_y, gpu, host_rows, need_gpu, quantize, sample_rows, say, to_dev,
                      weights, x_host)

pytestmark = gpu

FMTS = [synth.Q8_0, synth.Q4_K, synth.IQ4_XS, synth.Q5_K, synth.Q6_K, synth.Q8G128]
NAMES = {synth.Q8_0: "q8_0", synth.Q4_K: "q4_K", synth.IQ4_XS: "iq4_xs", synth.Q5_K: "q5_K", synth.Q6_K: "q6_K",
         synth.Q8G128: "q8g128"}
SENTINEL = -12345.0


def _case(fmt, rows, k, name):
    ws = [synth.make_weights(fmt, n, k, f"{name}/w{i}").data for i, n in enumerate(rows)]
    return ws, [to_dev(w) for w in ws]


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_batch_every_variant(fmt):
    qmv = need_gpu()
    k = 512 if fmt == synth.Q8_0 else 1024
    rows = [37, 100, 5, 64, 129]
    ws, wd = _case(fmt, rows, k, f"bv/{fmt}")
    x = x_host(16, k, f"bvx/{fmt}")
    res = [x_host(16, n, f"bvr/{fmt}/{i}") for i, n in enumerate(rows)]
    try:
        for v in range(len(qmv.variants())):
            qmv.set_tuning("variant", v)
            for t in (1, 2, 3, 5, 8, 13, 16):
                say(f"matvec_batch {NAMES[fmt]} variant {qmv.variant_name(v)} T={t}")
                xq = quantize(qmv, x[:t])
                ys = [torch.full((t, n + 3), SENTINEL, dtype=torch.float32, device="cuda") for n in rows]
                rs = [None, to_dev(res[1][:t]), None, None, None]
                ys[3][:, :rows[3]] = to_dev(res[3][:t])  # accumulate in place
                items = []
                for i, n in enumerate(rows):
                    r = ys[3][:, :] if i == 3 else rs[i]
                    items.append((wd[i], n, ys[i], r))
                qmv.matvec_batch(fmt, items, k, xq, t)
                qs, d, s = oracle.quantize_act(x[:t])
                for i, n in enumerate(rows):
                    r = res[i][:t] if i in (1, 3) else None
                    yr, mag = oracle.matvec(fmt, ws[i], k, qs, d, s, residual=r)
                    got = ys[i].cpu().numpy()
                    assert_y(got[:, :n], yr, mag, f"{NAMES[fmt]} v{v} T={t} item {i}")
                    assert np.all(got[:, n:] == SENTINEL), f"item {i}: columns past n_rows written"
    finally:
        qmv.set_tuning("variant", -1)


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_one_item_batch_is_matvec(fmt):
    qmv = need_gpu()
    n, k = 333, 2048
    w = weights(fmt, n, k, f"b1/{fmt}")
    for t in (1, 2, 4, 8, 16):
        say(f"one-item batch {NAMES[fmt]} T={t}")
        x = x_host(t, k, f"b1x/{fmt}/{t}")
        xq = quantize(qmv, x)
        y_mv = qmv.matvec(fmt, w, n, k, xq, t)
        (y_b,) = qmv.matvec_batch(fmt, [(w, n, None, None)], k, xq, t)
        r = to_dev(x_host(t, n, f"b1r/{fmt}/{t}"))
        (y_r,) = qmv.matvec_batch(fmt, [(w, n, None, r)], k, xq, t)
        torch.cuda.synchronize()
        assert torch.equal(y_b, y_mv), f"T={t}"
        assert torch.equal(y_r, y_mv + r), f"T={t}"


@pytest.mark.parametrize("fmt,n,k,tokens", [
    (synth.Q4_K, 14336, 4096, (1, 2, 4, 8, 16)),
    (synth.IQ4_XS, 4096, 14336, (1, 2, 16)),
], ids=["q4_K_gate_up_2x14336x4096", "iq4_xs_2x4096x14336"])
def test_batch_full_sibling_shapes(fmt, n, k, tokens):
    qmv = need_gpu()
    wd = [weights(fmt, n, k, f"sib/{fmt}/gate"), weights(fmt, n, k, f"sib/{fmt}/up")]
    rows = sample_rows(n, 96, f"sib/{fmt}/rows")
    wh = [host_rows(w, rows) for w in wd]
    for t in tokens:
        say(f"sibling batch {NAMES[fmt]} 2x{n}x{k} T={t}")
        x = x_host(t, k, f"sibx/{fmt}/{t}")
        xq = quantize(qmv, x)
        r = x_host(t, n, f"sibr/{fmt}/{t}")
        y0, y1 = qmv.matvec_batch(fmt, [(wd[0], n, None, None), (wd[1], n, None, to_dev(r))], k, xq, t)
        qs, d, s = oracle.quantize_act(x)
        yr0, m0 = oracle.matvec(fmt, wh[0], k, qs, d, s)
        yr1, m1 = oracle.matvec(fmt, wh[1], k, qs, d, s, residual=r[:, rows])
        assert_y(y0.cpu().numpy()[:, rows], yr0, m0, f"gate T={t}")
        assert_y(y1.cpu().numpy()[:, rows], yr1, m1, f"up + residual T={t}")


def test_batch_edges():
    """Eight items (the maximum) of one to 65 rows over Q8_0 k = 32, and an
    in-place residual applied twice."""
    qmv = need_gpu()
    fmt, k = synth.Q8_0, 32
    rows = [1, 2, 63, 64, 65, 1, 17, 3]
    ws, wd = _case(fmt, rows, k, "be")
    for t in (1, 4, 16):
        say(f"batch edges T={t}")
        x = x_host(t, k, f"bex/{t}")
        xq = quantize(qmv, x)
        ys = qmv.matvec_batch(fmt, [(w, n, None, None) for w, n in zip(wd, rows)], k, xq, t)
        qs, d, s = oracle.quantize_act(x)
        for i, n in enumerate(rows):
            yr, mag = oracle.matvec(fmt, ws[i], k, qs, d, s)
            assert_y(ys[i].cpu().numpy(), yr, mag, f"T={t} item {i}")
    # y <- W x + y, twice, from y0
    n, k = 300, 1024
    w = synth.make_weights(synth.Q4_K, n, k, "be/inplace").data
    x = x_host(2, k, "be/inplace/x")
    xq = quantize(qmv, x)
    y0 = x_host(2, n, "be/inplace/y0")
    y = to_dev(y0)
    wdev = to_dev(w)
    qs, d, s = oracle.quantize_act(x)
    expect = y0.astype(np.float32)
    for rep in range(2):
        say(f"in-place residual, call {rep}")
        qmv.matvec_batch(synth.Q4_K, [(wdev, n, y, y)], k, xq, 2)
        yr, mag = oracle.matvec(synth.Q4_K, w, k, qs, d, s, residual=expect)
        got = y.cpu().numpy()
        assert_y(got, yr, mag, f"in-place call {rep}")
        expect = got
