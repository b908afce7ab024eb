"""Edge shapes and values of qmv_matvec: one row, a few rows, ragged tails, a
single block of K, Q8_0 and Q8G128 rows whose blocks start at every alignment, all-zero
activations, the int8 weight value -128 (valid in Q8_0 but never drawn by the
generator), and zero sub-block scales."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_y, gpu, need_gpu, quantize, say, to_dev, x_host

pytestmark = gpu

FMTS = [synth.Q8_0, synth.Q4_K, synth.IQ4_XS, synth.Q5_K, synth.Q6_K, synth.Q8G128]


def _check(qmv, fmt, w, n, k, x, what):
    t = x.shape[0]
    say(f"edge {what} fmt={fmt} N={n} K={k} T={t}")
    xq = quantize(qmv, x)
    y = qmv.matvec(fmt, to_dev(w), n, k, xq, t).cpu().numpy()
    qs, d, s = oracle.quantize_act(x)
    yr, mag = oracle.matvec(fmt, w, k, qs, d, s)
    assert_y(y, yr, mag, what)
    got = qmv.block_dots(fmt, to_dev(w), n, k, xq, t).cpu().numpy()
    assert np.array_equal(got, oracle.block_dots(fmt, w, k, qs, s)), what


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [1, 3, 257])
def test_row_counts(fmt, n):
    qmv = need_gpu()
    k = 256
    for t in (1, 7, 16):
        w = synth.make_weights(fmt, n, k, f"edge/{fmt}/{n}").data
        _check(qmv, fmt, w, n, k, x_host(t, k, "edge/x"), f"rows {n}")


@pytest.mark.parametrize("k", [32, 64, 96, 160, 2080])
def test_q8_0_odd_block_counts(k):
    """Rows of 34-byte blocks: odd block counts make rows start 2 mod 4."""
    qmv = need_gpu()
    n = 45
    w = synth.make_weights(synth.Q8_0, n, k, f"edge/q8/{k}").data
    for t in (1, 3, 16):
        _check(qmv, synth.Q8_0, w, n, k, x_host(t, k, f"edge/q8x/{k}"), f"q8_0 K={k}")


@pytest.mark.parametrize("k", [128, 384, 640, 5120])
def test_q8g128_group_counts(k):
    """Rows of 130-byte groups: odd rows (and, with an odd group count, every
    other group) start 2 mod 4, so the quants of every unit are read both
    dword aligned and realigned; the int8 value -128 included."""
    qmv = need_gpu()
    n = 45
    w = synth.make_weights(synth.Q8G128, n, k, f"edge/q8g/{k}", q8_range=(-128, 127)).data
    for t in (1, 3, 16):
        _check(qmv, synth.Q8G128, w, n, k, x_host(t, k, f"edge/q8gx/{k}"), f"q8g128 K={k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_activations(fmt):
    qmv = need_gpu()
    n, k = 50, 512
    w = synth.make_weights(fmt, n, k, f"edge/z/{fmt}").data
    x = np.zeros((3, k), np.float32)
    x[1, 100] = 2.0  # one token with a single non-zero block
    _check(qmv, fmt, w, n, k, x, "zero x")


def test_q8_0_minus_128():
    qmv = need_gpu()
    n, k = 33, 1024
    wf = synth.make_weights(synth.Q8_0, n, k, "edge/m128", q8_range=(-128, 127), keep_fields=True)
    w = wf.data.copy()
    w.reshape(n, k // 32, 34)[:, :, 2:] = 0x80  # every quant -128
    w.reshape(n, k // 32, 34)[5, 3, 2:] = wf.q[5, 96:128].view(np.uint8)
    x = x_host(4, k, "edge/m128x")
    x[2, :32] = 127.0  # an activation block of all +127
    _check(qmv, synth.Q8_0, w, n, k, x, "q8_0 -128")


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.IQ4_XS, synth.Q5_K, synth.Q6_K])
def test_zero_and_extreme_scales(fmt):
    qmv = need_gpu()
    n, k = 20, 1024
    ns = k // 256
    q = synth.nibbles(synth.stream(f"edge/sc/{fmt}"), 0, n * k).reshape(n, k)
    d = synth.scale_f16(synth.stream(f"edge/scd/{fmt}"), 0, n * ns).reshape(n, ns)
    # raw 6-bit scales cover 0..63 (IQ4_XS 32 is an effective zero scale)
    sc = (np.arange(n * ns * 8) % 64).astype(np.uint8).reshape(n, ns, 8)
    if fmt == synth.Q6_K:  # every int8 scale (-128 included, never drawn) and 6-bit value
        q6 = synth.randint(synth.stream(f"edge/sc6/{fmt}"), 0, n * k, 0, 63).astype(np.uint8).reshape(n, k)
        sc6 = ((np.arange(n * ns * 16) % 256) - 128).astype(np.int8).reshape(n, ns, 16)
        q6[0, :64] = 0   # q - 32 = -32 throughout a block pair
        q6[1, :64] = 63  # q - 32 = +31
        w = synth.pack_q6_k(d, sc6, q6)
        for t in (1, 16):
            _check(qmv, fmt, w, n, k, x_host(t, k, f"edge/scx/{fmt}"), "scales")
        return
    if fmt == synth.Q5_K:  # 5-bit values: every fifth bit pattern
        q = synth.randint(synth.stream(f"edge/sc5/{fmt}"), 0, n * k, 0, 31).astype(np.uint8).reshape(n, k)
    if fmt in (synth.Q4_K, synth.Q5_K):
        m = sc[:, :, ::-1].copy()
        w = (synth.pack_q4_k if fmt == synth.Q4_K else synth.pack_q5_k)(d, d, sc, m, q)
    else:
        w = synth.pack_iq4_xs(d, sc, q)
    for t in (1, 16):
        _check(qmv, fmt, w, n, k, x_host(t, k, f"edge/scx/{fmt}"), "scales")


def test_stream_read_covers_every_byte():
    """The read hook loads every 16-byte piece, the ragged last workgroup's
    included: a piece whose dwords fold to the hook's key (and nothing else
    non-zero in that lane's loads) makes it store the key; otherwise it
    stores nothing."""
    qmv = need_gpu()
    key = 0x9E3779B9
    for nbytes in (16, 4096, 4096 * 3 + 48, 17825792):
        for piece in (0, nbytes // 16 - 1):
            say(f"stream_read bytes={nbytes} piece={piece}")
            t = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
            sink = qmv.stream_read(t)
            torch.cuda.synchronize()
            assert int(sink[0]) == 0
            t.view(torch.int32)[4 * piece + 1] = np.array(key, np.uint32).view(np.int32).item()
            sink = qmv.stream_read(t)
            torch.cuda.synchronize()
            assert np.array(int(sink[0]), np.int32).view(np.uint32) == key, (nbytes, piece)
