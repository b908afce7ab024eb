"""Pins of the CPU oracle against things other than itself.

  * hand-worked activation blocks (ties, zero block, single non-zero value);
  * quantizer invariants (argmax -> +-127, |x - d q| <= d/2, grid values
    re-quantize to themselves);
  * an integer special case that reduces to numpy's int64 matrix product
    exactly (unit weight scales, activations that are integers with amax 127);
  * brute force on tiny shapes: fp64 weights rebuilt from the generator's
    fields (never from the oracle's decoder) times dequantized activations;
  * the closed-form bound on the activation quantization error;
  * the routed (MoE) matvec against a loop of dense calls, token permutation,
    duplicate and dropped ids;
  * mutants: a copy of the oracle with one planted mistake must fail at least
    one of the pins above.
"""
import ctypes
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import synth
from golden_io import act_cases, codebook

CB = codebook()


# ------------------------------------------------------------------ pins
def pin_act_cases():
    for c in act_cases():
        qs, d, s = oracle.quantize_act(c["x"][None])
        assert qs[0].astype(np.int64).tolist() == c["q"].tolist(), c
        amax = np.float32(np.abs(c["x"]).max())
        assert d[0, 0] == np.float32(amax / np.float32(127.0))
        assert abs(float(d[0, 0]) - c["d"]) <= 1e-7 * max(1.0, c["d"])
        assert int(s[0, 0]) == c["s"]


def pin_act_invariants():
    x = synth.make_x(5, 1024, "inv") * np.float32(3.0)
    qs, d, s = oracle.quantize_act(x)
    xb = x.reshape(5, 32, 32).astype(np.float64)
    qb = qs.reshape(5, 32, 32).astype(np.int64)
    arg = np.abs(xb).argmax(-1)
    top = np.take_along_axis(qb, arg[..., None], -1)[..., 0]
    assert np.array_equal(np.abs(top), np.full_like(top, 127))
    assert np.array_equal(np.sign(top), np.sign(np.take_along_axis(xb, arg[..., None], -1)[..., 0]))
    err = np.abs(xb - d[..., None].astype(np.float64) * qb)
    assert np.all(err <= d[..., None].astype(np.float64) * (0.5 + 1e-5))
    assert np.array_equal(s, qb.sum(-1))
    # values on the grid of a block re-quantize to themselves
    grid = (d[..., None] * qb.astype(np.float32)).astype(np.float32).reshape(5, 1024)
    qs2, d2, _ = oracle.quantize_act(grid)
    assert np.array_equal(qs2, qs)


def _int_weights(fmt, n, k, seed):
    """Weights whose dequantized values are integers: every fp16 scale is 1."""
    if fmt in (synth.Q8_0, synth.Q8G128):
        q = synth.randint(synth.stream("iq", seed), 0, n * k, -127, 127).reshape(n, k)
        pack = synth.pack_q8_0 if fmt == synth.Q8_0 else synth.pack_q8g128
        data = pack(np.ones((n, k // synth.BLOCK_WEIGHTS[fmt]), np.float16), q.astype(np.int8))
        return data, q
    ns = k // 256
    if fmt == synth.Q6_K:  # int8 scale per 16 weights times (q - 32)
        q = synth.randint(synth.stream("iq6", seed), 0, n * k, 0, 63).reshape(n, k)
        sc = synth.randint(synth.stream("isc6", seed), 0, n * ns * 16, -127, 127).reshape(n, ns, 16)
        data = synth.pack_q6_k(np.ones((n, ns), np.float16), sc.astype(np.int8), q.astype(np.uint8))
        return data, np.repeat(sc, 16, axis=2).reshape(n, k) * (q - 32)
    q = synth.nibbles(synth.stream("iq", seed), 0, n * k).reshape(n, k).astype(np.int64)
    sc = synth.randint(synth.stream("isc", seed), 0, n * ns * 8, 0, 63).reshape(n, ns, 8)
    one = np.ones((n, ns), np.float16)
    j = np.repeat(sc, 32, axis=2).reshape(n, k)
    if fmt == synth.Q5_K:  # 5-bit values
        q = synth.randint(synth.stream("iq5", seed), 0, n * k, 0, 31).reshape(n, k).astype(np.int64)
    if fmt in (synth.Q4_K, synth.Q5_K):
        m = synth.randint(synth.stream("im", seed), 0, n * ns * 8, 0, 63).reshape(n, ns, 8)
        pack = synth.pack_q4_k if fmt == synth.Q4_K else synth.pack_q5_k
        data = pack(one, one, sc.astype(np.uint8), m.astype(np.uint8), q.astype(np.uint8))
        return data, j * q - np.repeat(m, 32, axis=2).reshape(n, k)
    data = synth.pack_iq4_xs(one, sc.astype(np.uint8), q.astype(np.uint8))
    return data, (j - 32) * CB[q]


def _int_acts(t, k, seed):
    """Integer activations whose every 32-block has amax exactly 127 (d = 1)."""
    x = synth.randint(synth.stream("ix", seed), 0, t * k, -126, 126).reshape(t, k // 32, 32)
    sign = np.where(synth.randint(synth.stream("isg", seed), 0, t * k // 32, 0, 1) > 0, 1, -1)
    x[:, :, 0] = 127 * sign.reshape(t, k // 32)
    return x.reshape(t, k)


def pin_integer_special_case():
    for fmt, k in ((synth.Q8_0, 96), (synth.Q4_K, 512), (synth.IQ4_XS, 768), (synth.Q5_K, 512),
                   (synth.Q6_K, 512), (synth.Q8G128, 384)):
        data, w_int = _int_weights(fmt, 7, k, seed=fmt)
        x = _int_acts(3, k, seed=fmt)
        qs, d, s = oracle.quantize_act(x.astype(np.float32))
        assert np.all(d == 1.0) and np.array_equal(qs.astype(np.int64), x)
        y, mag = oracle.matvec(fmt, data, k, qs, d, s)
        ref = x @ w_int.T  # numpy int64
        assert np.array_equal(y, ref.astype(np.float64)), fmt


def pin_residual():
    """Matvec + residual in the integer special case: y equals numpy's int64
    W x plus the (integer-valued, distinct per output) residual exactly, and
    the residual adds |r| to the tolerance magnitude."""
    for fmt, k in ((synth.Q8_0, 96), (synth.Q4_K, 512), (synth.IQ4_XS, 768), (synth.Q5_K, 512),
                   (synth.Q6_K, 512)):
        data, w_int = _int_weights(fmt, 7, k, seed=fmt)
        x = _int_acts(3, k, seed=fmt)
        qs, d, s = oracle.quantize_act(x.astype(np.float32))
        r = (np.arange(21, dtype=np.int64).reshape(3, 7) * 37 - 400)
        y, mag = oracle.matvec(fmt, data, k, qs, d, s, residual=r.astype(np.float32))
        y0, mag0 = oracle.matvec(fmt, data, k, qs, d, s)
        assert np.array_equal(y, (x @ w_int.T + r).astype(np.float64)), fmt
        assert np.array_equal(mag - mag0, np.abs(r).astype(np.float64)), fmt


def _dense_from_fields(wf):
    n, k = wf.data.shape[0], wf.k
    if wf.fmt in (synth.Q8_0, synth.Q8G128):
        return np.repeat(wf.d.astype(np.float64), synth.BLOCK_WEIGHTS[wf.fmt], axis=1) * wf.q.astype(np.float64)
    if wf.fmt == synth.Q6_K:
        g = np.repeat(wf.sc.astype(np.float64), 16, axis=2).reshape(n, k)
        return np.repeat(wf.d.astype(np.float64), 256, axis=1) * g * (wf.q.astype(np.float64) - 32)
    d = np.repeat(wf.d.astype(np.float64), 256, axis=1)
    sc = np.repeat(wf.sc.astype(np.float64), 32, axis=2).reshape(n, k)
    if wf.fmt in (synth.Q4_K, synth.Q5_K):
        dmin = np.repeat(wf.dmin.astype(np.float64), 256, axis=1)
        m = np.repeat(wf.m.astype(np.float64), 32, axis=2).reshape(n, k)
        return d * sc * wf.q - dmin * m
    return d * (sc - 32) * CB[wf.q.astype(np.int64)]


def pin_brute_force():
    for fmt, k in ((synth.Q8_0, 32), (synth.Q8_0, 256), (synth.Q4_K, 256), (synth.Q4_K, 512),
                   (synth.IQ4_XS, 256), (synth.IQ4_XS, 512), (synth.Q5_K, 256), (synth.Q5_K, 512),
                   (synth.Q6_K, 256), (synth.Q6_K, 512), (synth.Q8G128, 128), (synth.Q8G128, 640)):
        wf = synth.make_weights(fmt, 8, k, f"bf{fmt}", keep_fields=True)
        x = synth.make_x(3, k, f"bfx{fmt}")
        qs, d, s = oracle.quantize_act(x)
        y, mag = oracle.matvec(fmt, wf.data, k, qs, d, s)
        xdq = np.repeat(d.astype(np.float64), 32, axis=1) * qs.astype(np.float64)
        ref = xdq @ _dense_from_fields(wf).T
        assert np.all(np.abs(y - ref) <= 1e-12 * mag), fmt
        # the oracle's own dequantizer agrees with the fields as well
        assert np.allclose(oracle.dequant(fmt, wf.data, k), _dense_from_fields(wf), rtol=0, atol=1e-15)


def pin_quantization_bound():
    for fmt, k in ((synth.Q8_0, 512), (synth.Q4_K, 1024), (synth.IQ4_XS, 1024), (synth.Q5_K, 1024),
                   (synth.Q6_K, 1024), (synth.Q8G128, 1024)):
        wf = synth.make_weights(fmt, 6, k, f"qb{fmt}", keep_fields=True)
        x = synth.make_x(2, k, f"qbx{fmt}")
        qs, d, s = oracle.quantize_act(x)
        y, _ = oracle.matvec(fmt, wf.data, k, qs, d, s)
        w = _dense_from_fields(wf)
        exact = x.astype(np.float64) @ w.T
        bound = (np.abs(w)[None] * (np.repeat(d.astype(np.float64), 32, axis=1)[:, None] / 2)).sum(-1)
        assert np.all(np.abs(y - exact) <= bound * (1 + 1e-6) + 1e-12), fmt
        # and the bound is not vacuous: errors are a visible fraction of it
        assert np.abs(y - exact).max() > 1e-3 * bound.max()


def pin_moe_against_dense_loop():
    fmt, e, n, k, top_k = synth.IQ4_XS, 6, 5, 512, 3
    w = synth.make_weights(fmt, e * n, k, "moe/w").data
    ids = np.array([[0, 4, 2], [5, 5, 1], [3, -1, 6], [2, 0, 4]], np.int32)  # dup + dropped
    t = ids.shape[0]
    rw = np.array([[0.5, 0.25, 0.25], [0.1, 0.6, 0.3], [0.7, 0.2, 0.1], [0.3, 0.3, 0.4]], np.float32)
    for per_slot in (False, True):
        x = synth.make_x(t * top_k if per_slot else t, k, "moe/x")
        qs, d, s = oracle.quantize_act(x)
        ys, ms = oracle.moe_matvec(fmt, w, e, n, k, qs, d, s, ids, None, per_slot)
        yw, mw = oracle.moe_matvec(fmt, w, e, n, k, qs, d, s, ids, rw, per_slot)
        for ti in range(t):
            acc = np.zeros(n)
            for si in range(top_k):
                ex = int(ids[ti, si])
                xr = ti * top_k + si if per_slot else ti
                if 0 <= ex < e:
                    yd, md = oracle.matvec(fmt, w[ex * n:(ex + 1) * n], k,
                                           qs[xr:xr + 1], d[xr:xr + 1], s[xr:xr + 1])
                else:
                    yd, md = np.zeros((1, n)), np.zeros((1, n))
                assert np.array_equal(ys[ti, si], yd[0]) and np.array_equal(ms[ti, si], md[0])
                acc += np.float64(rw[ti, si]) * yd[0]
            assert np.allclose(yw[ti], acc, rtol=0, atol=1e-12 * (mw[ti].max() + 1))
    # permuting tokens permutes outputs
    x = synth.make_x(t, k, "moe/x")
    qs, d, s = oracle.quantize_act(x)
    perm = np.array([2, 0, 3, 1])
    y1, _ = oracle.moe_matvec(fmt, w, e, n, k, qs, d, s, ids, rw, False)
    y2, _ = oracle.moe_matvec(fmt, w, e, n, k, qs[perm], d[perm], s[perm], ids[perm], rw[perm], False)
    assert np.array_equal(y1[perm], y2)


def pin_swiglu():
    """SwiGLU against values and identities that do not restate its formula:
    the logistic function at 1 (sigma(1) = 0.7310585786300049, a tabulated
    constant), silu(0) = 0, silu(x) - silu(-x) = x (x sigma(x) + x sigma(-x)),
    linearity in the up half, silu(x) -> x and -> -0 far out."""
    n = 4
    gu = np.array([[1.0, 0.0, 3.0, -2.5, 1.0, 7.0, 1.0, 1.0]], np.float32)
    h = oracle.swiglu(gu, n)
    assert abs(h[0, 0] - 0.7310585786300049) < 1e-15
    assert h[0, 1] == 0.0
    g = synth.make_x(3, 64, "swiglu/g").astype(np.float32) * np.float32(4.0)
    u = synth.make_x(3, 64, "swiglu/u").astype(np.float32)
    ones = np.ones_like(g)
    hp = oracle.swiglu(np.concatenate([g, ones], 1), 64)
    hn = oracle.swiglu(np.concatenate([-g, ones], 1), 64)
    assert np.allclose(hp - hn, g.astype(np.float64), rtol=0, atol=1e-14 * (1 + np.abs(g).max()))
    hu = oracle.swiglu(np.concatenate([g, u], 1), 64)
    assert np.allclose(hu, hp * u.astype(np.float64), rtol=1e-15, atol=0)
    far = oracle.swiglu(np.array([[60.0, -800.0, 2.0, 5.0]], np.float32), 2)
    assert abs(far[0, 0] - 120.0) < 1e-12 and far[0, 1] == 0.0 and np.signbit(far[0, 1])
    # the gate/up halves are taken from their own columns of a wider row
    wide = np.concatenate([g, u, np.full_like(g, 9.0)], 1)
    assert np.array_equal(oracle.swiglu(wide, 64), hu)


def pin_router_topk():
    """Router + top-k against hand-built cases: one-hot router rows make the
    logits equal chosen values exactly; ties go to the lower expert; the
    weights are a softmax of the chosen logits (checked as ratios
    w_i / w_j = exp(l_i - l_j) and a sum of 1); numpy's int64 matrix product
    on integer inputs gives the logits exactly."""
    e, k = 8, 64
    wr = np.zeros((e, k), np.float32)
    for i in range(e):
        wr[i, i] = 1.0
    x = np.zeros((2, k), np.float32)
    x[0, :e] = [0.5, 3.0, -1.0, 3.0, 2.0, 0.0, 7.0, 2.0]
    x[1, :e] = [1.0] * e  # all tied: experts 0, 1, 2 in order
    ids, w, logits = oracle.router_topk(x, wr, 3)
    assert ids.tolist() == [[6, 1, 3], [0, 1, 2]]
    assert np.array_equal(logits[0], x[0, :e].astype(np.float64))
    assert abs(w[0].sum() - 1.0) < 1e-15 and np.allclose(w[1], 1.0 / 3.0, rtol=1e-15)
    assert abs(w[0, 0] / w[0, 1] - np.exp(4.0)) < 1e-12 and abs(w[0, 1] / w[0, 2] - 1.0) < 1e-15
    rng_x = synth.randint(synth.stream("router/x"), 0, 3 * k, -9, 9).reshape(3, k)
    rng_w = synth.randint(synth.stream("router/w"), 0, 16 * k, -9, 9).reshape(16, k)
    ids, w, logits = oracle.router_topk(rng_x.astype(np.float32), rng_w.astype(np.float32), 5)
    ref = rng_x.astype(np.int64) @ rng_w.astype(np.int64).T
    assert np.array_equal(logits, ref.astype(np.float64))
    for t in range(3):
        order = sorted(range(16), key=lambda i: (-ref[t, i], i))[:5]
        assert ids[t].tolist() == order
    # the selection from given logits agrees with the one from the matvec
    ids2, w2 = oracle.topk_from_logits(logits.astype(np.float32), 5)
    assert np.array_equal(ids2, ids) and np.allclose(w2, w, rtol=1e-15)


def pin_topk_from_logits_ties():
    """The selection from given fp32 logits, on hand-written cases whose
    answers are written out here: exact ties inside the picks and across the
    top-k boundary go to the lower expert index, -0 and +0 compare equal
    (so they are a tie as well), and the weights are a softmax of the chosen
    logits (equal for tied picks, ratios exp(l_i - l_j), sum 1)."""
    nz = np.float32(-0.0)
    logits = np.array([
        [2.0, 5.0, 5.0, -1.0, 5.0, 0.0, 0.0, 0.0],   # three-way tie at the top, ties at 0 below
        [1.0, 3.0, 3.0, 3.0, 0.0, 3.0, -2.0, 3.0],   # the boundary falls inside a five-way tie
        [nz, 0.0, nz, -3.0, 0.0, -1.0, nz, -0.5],    # signed zeros: all five are one tie
        [0.0, nz, 0.0, 1.0, nz, -7.0, 0.0, 0.5],
    ], np.float32)
    ids, w = oracle.topk_from_logits(logits, 6)
    assert ids.tolist() == [[1, 2, 4, 0, 5, 6],
                            [1, 2, 3, 5, 7, 0],
                            [0, 1, 2, 4, 6, 7],
                            [3, 7, 0, 1, 2, 4]]
    ids2, _ = oracle.topk_from_logits(logits, 2)
    assert ids2.tolist() == [[1, 2], [1, 2], [0, 1], [3, 7]]
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    # row 0 picks 5, 5, 5, 2, 0, 0: weights e^0, e^0, e^0, e^-3, e^-5, e^-5 over their sum
    z = np.array([1.0, 1.0, 1.0, np.exp(-3.0), np.exp(-5.0), np.exp(-5.0)])
    assert np.allclose(w[0], z / z.sum(), rtol=1e-15, atol=0)
    # row 2: five signed zeros and -0.5 -> five equal weights and one e^-0.5 times smaller
    assert np.allclose(w[2, :5], w[2, 0], rtol=0, atol=0)
    assert abs(w[2, 0] / w[2, 5] - np.exp(0.5)) < 1e-13
    # a single expert, and top_k equal to the expert count (a full ordering)
    one, w1 = oracle.topk_from_logits(np.array([[4.0]], np.float32), 1)
    assert one.tolist() == [[0]] and w1.tolist() == [[1.0]]
    full, _ = oracle.topk_from_logits(logits[1:2], 8)
    assert full.tolist() == [[1, 2, 3, 5, 7, 0, 4, 6]]


PINS = [pin_act_cases, pin_act_invariants, pin_integer_special_case, pin_residual, pin_brute_force,
        pin_quantization_bound, pin_moe_against_dense_loop, pin_swiglu, pin_router_topk,
        pin_topk_from_logits_ties]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_integer_partials_exact_formula_sizes():
    """Partials stay far inside int32 / fp32-exact range at the extremes."""
    k = 256
    # Q8_0 extreme: all +127 weights times all +127 activations
    w = synth.pack_q8_0(np.ones((1, 8), np.float16), np.full((1, k), 127, np.int8))
    x = np.full((1, k), 127.0, np.float32)
    qs, d, s = oracle.quantize_act(x)
    p = oracle.block_dots(synth.Q8_0, w, k, qs, s)
    assert np.all(p == 32 * 127 * 127)
    # IQ4_XS extreme: effective scale -32, codebook -127, activation +127
    w = synth.pack_iq4_xs(np.ones((1, 1), np.float16), np.zeros((1, 1, 8), np.uint8),
                          np.zeros((1, k), np.uint8))
    p = oracle.block_dots(synth.IQ4_XS, w, k, qs, s)
    assert np.all(p == -32 * 32 * -127 * 127) and abs(int(p.max())) < 2 ** 24


# --------------------------------------------------------------- mutants
MUTANTS = {
    "min_sign": ("double tm = -dm[b]", "double tm = dm[b]"),
    "min_dropped": ("acc += tp + tm;", "acc += tp;"),
    "q4k_nibble_swap": ("o->q[64 * c + i] = Q[32 * c + i] & 15;", "o->q[64 * c + i] = Q[32 * c + i] >> 4;"),
    "q4k_scale_hi_bits": ("((S[j - 4] >> 6) << 4)", "((S[j] >> 6) << 4)"),
    "q5k_high_bit_swapped": ("16 * ((H[i] >> (2 * c)) & 1);", "16 * ((H[i] >> (2 * c + 1)) & 1);"),
    "q5k_high_bit_dropped": ("hi + 16 * ((H[i] >> (2 * c + 1)) & 1);", "hi;"),
    "q6k_offset": ("blk.d * blk.sc[i / 16] * (blk.q[i] - 32)", "blk.d * blk.sc[i / 16] * (blk.q[i] - 31)"),
    "q6k_dot_offset": ("(blk.q[w] - 32) * qx[32 * b + i]", "(blk.q[w] - 31) * qx[32 * b + i]"),
    "q6k_scale_group": ("p += blk.sc[w / 16]", "p += blk.sc[w / 32]"),
    "q6k_high_bits": ("int two = (H[32 * h + l] >> (2 * j)) & 3;", "int two = (H[32 * h + l] >> j) & 3;"),
    "q6k_d_offset": ("fmt == FMT_Q6_K ? 208 : 0", "fmt == FMT_Q6_K ? 206 : 0"),
    "q8g128_group_of_64": ("half_to_double(rd16(row + (b / 4) * 130))", "half_to_double(rd16(row + (b / 2) * 130))"),
    "q8g128_quant_offset": ("i < 128; ++i) o->q[i] = (int8_t)b[2 + i];", "i < 128; ++i) o->q[i] = (int8_t)b[1 + i];"),
    "iq4_offset": ("(blk.ls[j] - 32) * p", "(blk.ls[j] - 31) * p"),
    "iq4_scales_h": ("(((sh >> (2 * j)) & 3) << 4)", "(((sh >> j) & 3) << 4)"),
    "iq4_nibble_half": ("o->idx[32 * j + 16 + i] = Q[16 * j + i] >> 4;", "o->idx[32 * j + 16 + i] = Q[16 * j + i] & 15;"),
    "codebook_entry": ("89,  113", "89,  112"),
    "round_half_even": ("(int)roundf(v)", "(int)rintf(v)"),
    "amax_signed": ("float a = fabsf(xb[i]);", "float a = xb[i];"),
    "q8_reversed_operand": ("p += blk.q[i] * qx[32 * b + i];", "p += blk.q[i] * qx[32 * b + 31 - i];"),
    "block_sum_dropped": ("sum += qi;", "sum += 0;"),
    "fp16_exponent": ("e - 25", "e - 24"),
    "silu_sign": ("exp(-g);  /*", "exp(g);  /*"),
    "swiglu_up_column": ("gu[r * ldg + n_ff + i]", "gu[r * ldg + i]"),
    "topk_tie_upper": ("if (best < 0 || l[e] > l[best]) best = e;  /* strict", "if (best < 0 || l[e] >= l[best]) best = e;  /* strict"),
    "logits_topk_tie_upper": ("l[e] > l[best]) best = e;\n", "l[e] >= l[best]) best = e;\n"),
    "logits_topk_signed_zero": ("l[e] > l[best]) best = e;\n",
                                "l[e] > l[best] || (l[e] == l[best] && signbit(l[best]) && !signbit(l[e]))) best = e;\n"),
    "logits_softmax_unnormalized": ("exp((double)l[ids[t * top_k + j]] - m) / sum;",
                                    "exp((double)l[ids[t * top_k + j]] - m);"),
    "softmax_unnormalized": ("w[t * top_k + j] = exp(l[ids[t * top_k + j]] - m) / sum;\n  }\n  return 0;\n}\n\n/* The selection", "w[t * top_k + j] = exp(l[ids[t * top_k + j]] - m);\n  }\n  return 0;\n}\n\n/* The selection"),
    "residual_dropped": ("y[t * n_rows + n] += rv;", "y[t * n_rows + n] += 0.0;"),
    "residual_columns_reversed": ("(double)res[t * ldr + n];", "(double)res[t * ldr + n_rows - 1 - n];"),
    "router_transposed": ("acc += (double)wr[e * k + i] * (double)x[t * ldx + i];", "acc += (double)wr[i * n_experts + e] * (double)x[t * ldx + i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mut.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib_path = os.path.join(tmp, "libmut.so")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                        "-o", lib_path, path, "-lm"], check=True)
        saved = oracle._lib
        oracle._lib = None
        real_lib = oracle._LIB
        try:
            oracle._LIB = lib_path
            oracle._load()
            failed = []
            for pin in PINS:
                try:
                    pin()
                except AssertionError:
                    failed.append(pin.__name__)
            assert failed, f"mutant {name} passed every pin"
        finally:
            oracle._LIB = real_lib
            oracle._lib = saved
