"""Block formats: hand-assembled byte images, exhaustive field packing round
trips and weight-order ramps between the generator's packer and the oracle's
decoders, and the IQ4_XS codebook invariants."""
import numpy as np
import pytest

import oracle
import synth
from golden_io import codebook, hand_blocks


def _f16(v):
    return np.array(v, dtype=np.float16)


def _pattern_q():
    return np.array([(k + k // 16) % 16 for k in range(256)], dtype=np.uint8)


def test_hand_block_q8_0():
    blk = hand_blocks()["q8_0"]
    d = _f16([[blk["d"][0]]])
    q = np.array([blk["q"]], dtype=np.int8)
    assert synth.pack_q8_0(d, q).tobytes() == blk["hex"]
    f = oracle.unpack(synth.Q8_0, np.frombuffer(blk["hex"], np.uint8), 32)
    assert f["d"][0, 0] == 0.5 and f["q"][0].tolist() == [int(v) for v in blk["q"]]
    w = oracle.dequant(synth.Q8_0, np.frombuffer(blk["hex"], np.uint8), 32)
    assert w[0].tolist() == [(i - 16) / 2 for i in range(32)]


def test_hand_block_q4_k():
    blk = hand_blocks()["q4_k"]
    q = _pattern_q()[None]
    sc = np.array([[blk["sc"]]], dtype=np.uint8)
    m = np.array([[blk["m"]]], dtype=np.uint8)
    packed = synth.pack_q4_k(_f16([[blk["d"][0]]]), _f16([[blk["dmin"][0]]]), sc, m, q)
    assert packed.tobytes() == blk["hex"]
    f = oracle.unpack(synth.Q4_K, np.frombuffer(blk["hex"], np.uint8), 256)
    assert f["d"][0, 0] == 1.0 and f["dmin"][0, 0] == 0.5
    assert f["sc"][0, 0].tolist() == [int(v) for v in blk["sc"]]
    assert f["m"][0, 0].tolist() == [int(v) for v in blk["m"]]
    assert np.array_equal(f["q"][0], q[0])
    # weight = d * sc_j * q - dmin * m_j, with j = k // 32
    w = oracle.dequant(synth.Q4_K, np.frombuffer(blk["hex"], np.uint8), 256)[0]
    j = np.arange(256) // 32
    assert np.array_equal(w, 1.0 * np.array(blk["sc"])[j] * q[0] - 0.5 * np.array(blk["m"])[j])


def test_hand_block_q5_k():
    blk = hand_blocks()["q5_k"]
    q = np.array([[(k + k // 16) % 32 for k in range(256)]], dtype=np.uint8)
    sc = np.array([[blk["sc"]]], dtype=np.uint8)
    m = np.array([[blk["m"]]], dtype=np.uint8)
    packed = synth.pack_q5_k(_f16([[blk["d"][0]]]), _f16([[blk["dmin"][0]]]), sc, m, q)
    assert packed.tobytes() == blk["hex"]
    f = oracle.unpack(synth.Q5_K, np.frombuffer(blk["hex"], np.uint8), 256)
    assert f["d"][0, 0] == 1.0 and f["dmin"][0, 0] == 0.5
    assert f["sc"][0, 0].tolist() == [int(v) for v in blk["sc"]]
    assert f["m"][0, 0].tolist() == [int(v) for v in blk["m"]]
    assert np.array_equal(f["q"][0], q[0])
    w = oracle.dequant(synth.Q5_K, np.frombuffer(blk["hex"], np.uint8), 256)[0]
    j = np.arange(256) // 32
    assert np.array_equal(w, 1.0 * np.array(blk["sc"])[j] * q[0] - 0.5 * np.array(blk["m"])[j])
    # the header and the nibble bytes are those of the q4_K block with q % 16
    q4 = hand_blocks()["q4_k"]["hex"]
    assert blk["hex"][:16] == q4[:16] and blk["hex"][48:] == q4[16:]


def test_hand_block_q6_k():
    blk = hand_blocks()["q6_k"]
    q = np.array([[(k + k // 16) % 64 for k in range(256)]], dtype=np.uint8)
    sc = np.array([[blk["sc"]]], dtype=np.int8)
    packed = synth.pack_q6_k(_f16([[blk["d"][0]]]), sc, q)
    assert packed.tobytes() == blk["hex"]
    f = oracle.unpack(synth.Q6_K, np.frombuffer(blk["hex"], np.uint8), 256)
    assert f["d"][0, 0] == 0.5
    assert f["sc"][0, 0].tolist() == [int(v) for v in blk["sc"]]
    assert np.array_equal(f["q"][0], q[0])
    # weight = d * scales[k // 16] * (q - 32)
    w = oracle.dequant(synth.Q6_K, np.frombuffer(blk["hex"], np.uint8), 256)[0]
    g = np.arange(256) // 16
    assert np.array_equal(w, 0.5 * np.array(blk["sc"])[g] * (q[0].astype(np.float64) - 32))


def test_hand_block_q8g128():
    blk = hand_blocks()["q8g128"]
    q = np.array([[i - 64 for i in range(128)]], dtype=np.int8)
    assert synth.pack_q8g128(_f16([[blk["d"][0]]]), q).tobytes() == blk["hex"]
    f = oracle.unpack(synth.Q8G128, np.frombuffer(blk["hex"], np.uint8), 128)
    assert f["d"][0, 0] == 0.5 and f["q"][0].tolist() == q[0].tolist()
    w = oracle.dequant(synth.Q8G128, np.frombuffer(blk["hex"], np.uint8), 128)
    assert w[0].tolist() == [(i - 64) / 2 for i in range(128)]


def test_q8g128_group_scales_in_order():
    """Three groups with scales 1, 2, 4: each weight takes its own group's."""
    q = np.ones((1, 384), np.int8)
    w = oracle.dequant(synth.Q8G128, synth.pack_q8g128(_f16([[1.0, 2.0, 4.0]]), q), 384)[0]
    assert w.tolist() == [1.0] * 128 + [2.0] * 128 + [4.0] * 128


def test_hand_block_iq4_xs():
    blk = hand_blocks()["iq4_xs"]
    q = _pattern_q()[None]
    ls = np.array([[blk["ls"]]], dtype=np.uint8)
    packed = synth.pack_iq4_xs(_f16([[blk["d"][0]]]), ls, q)
    assert packed.tobytes() == blk["hex"]
    f = oracle.unpack(synth.IQ4_XS, np.frombuffer(blk["hex"], np.uint8), 256)
    assert f["sc"][0, 0].tolist() == [int(v) for v in blk["ls"]]
    assert np.array_equal(f["q"][0], q[0])
    w = oracle.dequant(synth.IQ4_XS, np.frombuffer(blk["hex"], np.uint8), 256)[0]
    j = np.arange(256) // 32
    cb = codebook()
    assert np.array_equal(w, (np.array(blk["ls"])[j] - 32) * cb[q[0]].astype(np.float64))


def test_q4_k_scale_min_packing_exhaustive():
    """Every (scale, min) pair in 0..63 x 0..63 at every one of the 8 positions."""
    v = np.arange(64 * 64)
    rng_fill = synth.randint(synth.stream("fill"), 0, 8 * 4096 * 8 * 2, 0, 63).reshape(8, 4096, 2, 8)
    for j in range(8):
        sc = rng_fill[j, :, 0].astype(np.uint8).reshape(4096, 1, 8)
        m = rng_fill[j, :, 1].astype(np.uint8).reshape(4096, 1, 8)
        sc[:, 0, j] = v // 64
        m[:, 0, j] = v % 64
        d = np.ones((4096, 1), np.float16)
        q = np.zeros((4096, 256), np.uint8)
        data = synth.pack_q4_k(d, d, sc, m, q)
        f = oracle.unpack(synth.Q4_K, data, 256)
        assert np.array_equal(f["sc"].astype(np.uint8), sc)
        assert np.array_equal(f["m"].astype(np.uint8), m)
        # and bytes -> fields -> bytes
        again = synth.pack_q4_k(d, d, f["sc"].astype(np.uint8), f["m"].astype(np.uint8), q)
        assert np.array_equal(again, data)


def test_iq4_xs_scale_packing_exhaustive():
    fill = synth.randint(synth.stream("fill2"), 0, 8 * 64 * 8, 0, 63).reshape(8, 64, 1, 8)
    for j in range(8):
        ls = fill[j].astype(np.uint8)
        ls[:, 0, j] = np.arange(64)
        d = np.ones((64, 1), np.float16)
        q = np.zeros((64, 256), np.uint8)
        data = synth.pack_iq4_xs(d, ls, q)
        f = oracle.unpack(synth.IQ4_XS, data, 256)
        assert np.array_equal(f["sc"].astype(np.uint8), ls)
        assert np.array_equal(synth.pack_iq4_xs(d, f["sc"].astype(np.uint8), q), data)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.IQ4_XS, synth.Q5_K, synth.Q6_K])
def test_weight_order_ramp(fmt):
    """A ramp of weight values survives pack -> oracle decode in weight order."""
    k = 512
    span = {synth.Q5_K: 32, synth.Q6_K: 64}.get(fmt, 16)
    q = np.array([[(7 * i + r) % span for i in range(k)] for r in range(3)], np.uint8)
    d = np.ones((3, 2), np.float16)
    sc = np.ones((3, 2, 8), np.uint8)
    if fmt == synth.Q4_K:
        data = synth.pack_q4_k(d, d, sc, sc, q)
    elif fmt == synth.Q5_K:
        data = synth.pack_q5_k(d, d, sc, sc, q)
    elif fmt == synth.Q6_K:
        data = synth.pack_q6_k(d, np.ones((3, 2, 16), np.int8), q)
    else:
        data = synth.pack_iq4_xs(d, sc, q)
    f = oracle.unpack(fmt, data, k)
    assert np.array_equal(f["q"], q)


def test_q8_0_fields_round_trip():
    wf = synth.make_weights(synth.Q8_0, 5, 320, "r", keep_fields=True)
    f = oracle.unpack(synth.Q8_0, wf.data, 320)
    assert np.array_equal(f["q"], wf.q.astype(np.int32))
    assert np.array_equal(f["d"], wf.d.astype(np.float64))


def test_fp16_decoder_all_finite_values():
    """The oracle's own binary16 decoder agrees with numpy on every finite fp16."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    fin = np.isfinite(vals)
    bits = bits[fin]
    n = bits.size
    blocks = np.zeros((n, 34), np.uint8)
    blocks[:, 0] = bits & 0xFF
    blocks[:, 1] = bits >> 8
    blocks[:, 2] = 1  # q[0] = 1 so the dequantized weight is d itself
    w = oracle.dequant(synth.Q8_0, blocks, 32)
    assert np.array_equal(w[:, 0], vals[fin].astype(np.float64))


def test_codebook_invariants():
    cb = codebook()
    assert np.all(np.diff(cb) > 0), "strictly increasing"
    assert cb.min() >= -128 and cb.max() <= 127
    # decode(i) == CB[i] through the oracle: d = 1, raw scale 33 (effective 1)
    q = np.tile(np.arange(16, dtype=np.uint8), 16)[None]
    data = synth.pack_iq4_xs(np.ones((1, 1), np.float16), np.full((1, 1, 8), 33, np.uint8), q)
    w = oracle.dequant(synth.IQ4_XS, data, 256)[0]
    assert np.array_equal(w, cb[q[0]].astype(np.float64))
    # round trip: the nearest codebook entry to a decoded value is its own index
    for i in range(16):
        assert int(np.argmin(np.abs(cb - w[i]))) == i
