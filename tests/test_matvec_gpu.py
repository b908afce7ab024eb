"""qmv_matvec and qmv_block_dots against the oracle.

  * integer partials of every 32-block: bit-exact (qmv_block_dots runs the
    same device decode and dot routines as the matvec kernels);
  * y: within 1e-4 of the sum of |per-block terms| of each output;
  * small shapes at every token count 1..16 and every kernel variant, with
    several row tiles and a ragged tail; the full workload shapes at their
    token counts on sampled rows, in the launch configuration the bench
    times.
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


def _oracle_y(fmt, w_host, k, x):
    qs, d, s = oracle.quantize_act(x)
    return oracle.matvec(fmt, w_host, k, qs, d, s)


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_block_dots_small(fmt):
    qmv = need_gpu()
    for n, k, t in ((37, 512, 3), (5, 256, 16), (64, 1024, 1)):
        say(f"block_dots {NAMES[fmt]} N={n} K={k} T={t}")
        w = synth.make_weights(fmt, n, k, f"bd/{fmt}/{n}").data
        x = x_host(t, k, f"bdx/{fmt}/{k}")
        xq = quantize(qmv, x)
        got = qmv.block_dots(fmt, to_dev(w), n, k, xq, t).cpu().numpy()
        qs, _, s = oracle.quantize_act(x)
        ref = oracle.block_dots(fmt, w, k, qs, s)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_every_token_count_and_variant(fmt):
    """N = 333 rows (several tiles of every variant plus a ragged tail)."""
    qmv = need_gpu()
    n = 333
    k = 1024 if fmt == synth.Q8_0 else 2048
    w = synth.make_weights(fmt, n, k, f"tv/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"tvx/{fmt}")
    try:
        for v in range(len(qmv.variants())):
            qmv.set_tuning("variant", v)
            for t in range(1, 17):
                say(f"matvec {NAMES[fmt]} variant {qmv.variant_name(v)} T={t}")
                xq = quantize(qmv, x[:t])
                y = qmv.matvec(fmt, wd, n, k, xq, t).cpu().numpy()
                yr, mag = _oracle_y(fmt, w, k, x[:t])
                assert_y(y, yr, mag, f"{NAMES[fmt]} v{v} T={t}")
    finally:
        qmv.set_tuning("variant", -1)


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_chunked_variants_long_k(fmt):
    """The LDS-chunked multi-token kernels on a row several chunks long
    (K = 14336 at 16 tokens), with a ragged token count and row tail."""
    qmv = need_gpu()
    n, k = 77, 14336
    w = synth.make_weights(fmt, n, k, f"lk/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"lkx/{fmt}")
    chunked = [v for v in range(len(qmv.variants()))
               if qmv.variant_name(v).startswith(("mt_", "mx_", "mf_"))]
    assert chunked
    try:
        for v in chunked:
            qmv.set_tuning("variant", v)
            for t in (16, 5, 2):
                say(f"matvec long K {NAMES[fmt]} variant {qmv.variant_name(v)} T={t}")
                xq = quantize(qmv, x[:t])
                y = qmv.matvec(fmt, wd, n, k, xq, t).cpu().numpy()
                yr, mag = _oracle_y(fmt, w, k, x[:t])
                assert_y(y, yr, mag, f"{NAMES[fmt]} {qmv.variant_name(v)} T={t}")
    finally:
        qmv.set_tuning("variant", -1)


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_long_row_kernel(fmt):
    """The long-row variants on rows longer than one pass of a workgroup's
    waves (K = 32768: several chunks per wave for the four- and eight-wave
    variants), an odd row count (the two-row variant's last group half
    empty), one to four tokens, and five (more than its registers hold: the
    multi-token kernel runs instead)."""
    qmv = need_gpu()
    n, k = 37, 32768
    w = synth.make_weights(fmt, n, k, f"lr/{fmt}").data
    wd = to_dev(w)
    x = x_host(5, k, f"lrx/{fmt}")
    long_rows = [v for v in range(len(qmv.variants())) if qmv.variant_name(v).startswith("lk_")]
    assert long_rows
    try:
        for t in (1, 2, 3, 4, 5):
            xq = quantize(qmv, x[:t])
            yr, mag = _oracle_y(fmt, w, k, x[:t])
            for v in long_rows:
                qmv.set_tuning("variant", v)
                say(f"matvec long rows {NAMES[fmt]} variant {qmv.variant_name(v)} T={t}")
                y = qmv.matvec(fmt, wd, n, k, xq, t).cpu().numpy()
                assert_y(y, yr, mag, f"{NAMES[fmt]} {qmv.variant_name(v)} T={t}")
    finally:
        qmv.set_tuning("variant", -1)


FULL = [
    ("q8_0_4096x4096", synth.Q8_0, 4096, 4096, (1,)),
    ("q4_k_14336x4096", synth.Q4_K, 14336, 4096, (1, 2, 4, 8, 16)),
    ("iq4_xs_4096x14336", synth.IQ4_XS, 4096, 14336, (1, 2, 4, 8, 16)),
    ("q8_0_head_152064x5120", synth.Q8_0, 152064, 5120, (1, 2, 4, 8, 16)),
    ("q5_k_14336x4096", synth.Q5_K, 14336, 4096, (1, 2, 4, 8, 16)),
    ("q6_k_14336x4096", synth.Q6_K, 14336, 4096, (1, 2, 4, 8, 16)),
    ("q8g128_head_152064x5120", synth.Q8G128, 152064, 5120, (1, 2, 4, 8, 16)),
    # other shapes whose automatic choice differs (rows per compute unit, row length)
    ("q4_k_28672x4096", synth.Q4_K, 28672, 4096, (4, 6, 16)),
    ("iq4_xs_28672x4096", synth.IQ4_XS, 28672, 4096, (4, 6, 16)),
    ("q4_k_8192x14336", synth.Q4_K, 8192, 14336, (2, 6, 16)),
    ("iq4_xs_8192x14336", synth.IQ4_XS, 8192, 14336, (4, 10, 16)),
    ("iq4_xs_4096x4096", synth.IQ4_XS, 4096, 4096, (3, 6, 16)),
    ("q4_k_8192x4096", synth.Q4_K, 8192, 4096, (4, 12)),
    ("q8_0_8192x4096", synth.Q8_0, 8192, 4096, (6, 16)),
    ("q8_0_4096x14336", synth.Q8_0, 4096, 14336, (3, 16)),
    ("q5_k_4096x14336", synth.Q5_K, 4096, 14336, (1, 4, 16)),
    ("q6_k_4096x14336", synth.Q6_K, 4096, 14336, (1, 4, 16)),
    ("q5_k_4096x4096", synth.Q5_K, 4096, 4096, (2, 8, 16)),
    # few rows, long K: the long-row kernel (sixteen or eight waves per row)
    ("q8_0_splitk_256x65536", synth.Q8_0, 256, 65536, (1, 2, 4)),
    ("q4_k_256x32768", synth.Q4_K, 256, 32768, (1, 2)),
]


@pytest.mark.parametrize("name,fmt,n,k,tokens", FULL, ids=[c[0] for c in FULL])
def test_full_shapes(name, fmt, n, k, tokens):
    qmv = need_gpu()
    say(f"full {name}: generating weights")
    wd = weights(fmt, n, k, f"{name}/W")
    rows = sample_rows(n, 640, f"rows/{name}")
    w_rows = host_rows(wd, rows)
    # the device generator agrees with the numpy generator on these rows
    for r in (rows[0], rows[len(rows) // 2], rows[-1]):
        ref = synth.make_weights(fmt, n, k, f"{name}/W", rows=(int(r), int(r) + 1)).data
        assert np.array_equal(w_rows[np.searchsorted(rows, r)], ref[0])
    x = x_host(max(tokens), k, f"{name}/x")
    # the bench's launch configuration: a split-K workspace where the shape takes one
    wsb = qmv.matvec_workspace_bytes(fmt, n, k, max(tokens))
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    for t in tokens:
        say(f"full {name} T={t}")
        xq = quantize(qmv, x[:t])
        y = qmv.matvec(fmt, wd, n, k, xq, t, ws=ws).cpu().numpy()
        yr, mag = _oracle_y(fmt, w_rows, k, x[:t])
        assert_y(y[:, rows], yr, mag, f"{name} T={t}")
        # exact integer partials on a few aligned row ranges
        rb = qmv.row_bytes(fmt, k)
        for r0 in (0, (n // 2) & ~7, n - 8):
            wsub = wd.view(-1)[r0 * rb:(r0 + 8) * rb]
            got = qmv.block_dots(fmt, wsub, 8, k, xq, t).cpu().numpy()
            qs, _, s = oracle.quantize_act(x[:t])
            ref = oracle.block_dots(fmt, wsub.cpu().numpy(), k, qs, s)
            assert np.array_equal(got, ref), (name, t, r0)


def test_head_every_token_count_on_row_slice():
    """The head at T = 1..16 on a 4096-row slice of its rows (K = 5120)."""
    qmv = need_gpu()
    n, k = 4096, 5120
    wd = weights(synth.Q8_0, n, k, "q8_0_head_152064x5120/W")
    w = wd.cpu().numpy()
    x = x_host(16, k, "q8_0_head_152064x5120/x")
    for t in range(1, 17):
        say(f"head slice T={t}")
        xq = quantize(qmv, x[:t])
        y = qmv.matvec(synth.Q8_0, wd, n, k, xq, t).cpu().numpy()
        yr, mag = _oracle_y(synth.Q8_0, w, k, x[:t])
        assert_y(y, yr, mag, f"head slice T={t}")


@pytest.mark.parametrize("fmt", FMTS, ids=[NAMES[f] for f in FMTS])
def test_iq4_and_q4k_every_token_count_config_k(fmt):
    """Every T = 1..16 at the workload's reduction length on a row slice."""
    qmv = need_gpu()
    k = {synth.Q8_0: 4096, synth.Q4_K: 4096, synth.IQ4_XS: 14336, synth.Q5_K: 4096, synth.Q6_K: 4096,
         synth.Q8G128: 5120}[fmt]
    n = 700
    w = synth.make_weights(fmt, n, k, f"tk/{fmt}").data
    wd = to_dev(w)
    x = x_host(16, k, f"tkx/{fmt}")
    for t in range(1, 17):
        xq = quantize(qmv, x[:t])
        y = qmv.matvec(fmt, wd, n, k, xq, t).cpu().numpy()
        yr, mag = _oracle_y(fmt, w, k, x[:t])
        assert_y(y, yr, mag, f"{NAMES[fmt]} K={k} T={t}")


def test_output_stride_leaves_padding():
    qmv = need_gpu()
    fmt, n, k, t = synth.IQ4_XS, 100, 512, 4
    w = synth.make_weights(fmt, n, k, "ld/w").data
    x = x_host(t, k, "ld/x")
    y = torch.full((t, n + 28), 7.0, dtype=torch.float32, device="cuda")
    qmv.matvec(fmt, to_dev(w), n, k, quantize(qmv, x), t, y=y)
    yh = y.cpu().numpy()
    yr, mag = _oracle_y(fmt, w, k, x)
    assert_y(yh[:, :n], yr, mag, "ldy")
    assert np.all(yh[:, n:] == 7.0)


def test_reuses_one_activation_buffer_across_formats():
    """One Q8 activation buffer serves every weight type."""
    qmv = need_gpu()
    k, t = 4096, 3
    x = x_host(t, k, "reuse/x")
    xq = quantize(qmv, x)
    for fmt in FMTS:
        w = synth.make_weights(fmt, 96, k, f"reuse/{fmt}").data
        y = qmv.matvec(fmt, to_dev(w), 96, k, xq, t).cpu().numpy()
        yr, mag = _oracle_y(fmt, w, k, x)
        assert_y(y, yr, mag, f"reuse {NAMES[fmt]}")
