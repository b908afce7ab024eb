"""Seeded generator: determinism, independence of row ranges, value ranges."""
import numpy as np
import pytest

import synth


def test_same_seed_same_bytes():
    a = synth.make_weights(synth.Q4_K, 8, 512, "C/W").data
    b = synth.make_weights(synth.Q4_K, 8, 512, "C/W").data
    assert np.array_equal(a, b)


def test_streams_and_seeds_differ():
    a = synth.make_weights(synth.IQ4_XS, 4, 256, "C/W").data
    b = synth.make_weights(synth.IQ4_XS, 4, 256, "C/V").data
    c = synth.make_weights(synth.IQ4_XS, 4, 256, "C/W", seed=1).data
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


@pytest.mark.parametrize("fmt,k", [(synth.Q8_0, 96), (synth.Q4_K, 512), (synth.IQ4_XS, 768), (synth.Q5_K, 512),
                                   (synth.Q6_K, 512), (synth.Q8G128, 384)])
def test_row_ranges_match_full_generation(fmt, k):
    full = synth.make_weights(fmt, 13, k, "C/W").data
    part = synth.make_weights(fmt, 13, k, "C/W", rows=(5, 11)).data
    assert np.array_equal(full[5:11], part)


@pytest.mark.parametrize("fmt,k", [(synth.Q8_0, 96), (synth.Q4_K, 512), (synth.IQ4_XS, 768), (synth.Q5_K, 512),
                                   (synth.Q6_K, 512), (synth.Q8G128, 384)])
def test_torch_generator_matches_numpy(fmt, k):
    from synth.device import make_weights_t
    ref = synth.make_weights(fmt, 11, k, "C/T").data
    got = make_weights_t(fmt, 11, k, "C/T", device="cpu", chunk_elems=3 * k).numpy()
    assert np.array_equal(got, ref)


def test_x_prefix_stable_across_token_counts():
    x4 = synth.make_x(4, 64, "x")
    x2 = synth.make_x(2, 64, "x")
    assert np.array_equal(x4[:2], x2)


def test_draw_ranges_and_moments():
    st = synth.stream("moments")
    r = synth.randint(st, 0, 200_000, -127, 127)
    assert r.min() == -127 and r.max() == 127
    assert abs(r.mean()) < 5 * 73.6 / np.sqrt(r.size)
    nib = synth.nibbles(st, 3, 100_000)
    assert nib.min() == 0 and nib.max() == 15
    assert abs(nib.mean() - 7.5) < 5 * 4.61 / np.sqrt(nib.size)
    z = synth.normal_f32(st, 0, 200_000).astype(np.float64)
    assert abs(z.mean()) < 5 / np.sqrt(z.size)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / z.size)
    s = synth.scale_f16(st, 0, 10_000).astype(np.float64)
    assert s.min() >= 1e-3 * (1 - 2 ** -10) and s.max() <= 1e-2 * (1 + 2 ** -10)


def test_offset_draws_are_consistent():
    st = synth.stream("off")
    assert np.array_equal(synth.randint(st, 0, 40, 0, 63)[7:29], synth.randint(st, 7, 22, 0, 63))
    assert np.array_equal(synth.nibbles(st, 0, 100)[13:77], synth.nibbles(st, 13, 64))
    assert np.array_equal(synth.normal_f32(st, 0, 20)[3:9], synth.normal_f32(st, 3, 6))


def test_routing_distinct_in_range_and_normalized():
    ids, rw = synth.make_routing(64, 128, 8, "moe")
    assert ids.shape == (64, 8) and rw.shape == (64, 8)
    assert ids.min() >= 0 and ids.max() < 128
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8
    assert np.allclose(rw.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert (rw > 0).all()
