"""The seeded input generator: published SplitMix64 outputs, determinism, slicing, moments."""
import math

import numpy as np

import synth


def test_splitmix64_published_outputs():
    # First outputs of the reference SplitMix64 generator (Vigna, splitmix64.c) from seed 1234567.
    got = [int(x) for x in synth.splitmix64_sequence(1234567, 5)]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_deterministic_and_seed_dependent():
    a = synth.normal(0, 1, (4096,), 1.0, "f32")
    b = synth.normal(0, 1, (4096,), 1.0, "f32")
    c = synth.normal(1, 1, (4096,), 1.0, "f32")
    d = synth.normal(0, 2, (4096,), 1.0, "f32")
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_slice_equals_whole():
    B, H, N, D = 2, 3, 50, 8
    whole = synth.normal(0, 2, (B, H, N, D), D ** -0.5, "bf16")
    for b in range(B):
        for h in range(H):
            part = synth.pair_slice(0, 2, B, H, N, D, b, h, "bf16")
            assert np.array_equal(part, whole[b, h])
            mid = synth.pair_slice(0, 2, B, H, N, D, b, h, "bf16", 10, 37)
            assert np.array_equal(mid, whole[b, h, 10:37])


def test_rounding_chain():
    x64 = synth.normal(3, 1, (10000,), 0.125, "f64")
    x32 = synth.normal(3, 1, (10000,), 0.125, "f32")
    xbf = synth.normal(3, 1, (10000,), 0.125, "bf16")
    assert np.array_equal(x32, x64.astype(np.float32))
    assert np.array_equal(xbf, synth.f32_to_bf16_bits(x32))
    back = synth.bf16_bits_to_f64(xbf)
    assert np.all(np.abs(back - x32) <= np.abs(x32) * 2.0 ** -8 + 1e-30)


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9, -2.5, 0.0],
                    dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6); 1+2^-7+2^-9 rounds down.
    expect = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 0.0])
    np.testing.assert_array_equal(synth.bf16_bits_to_f64(bits), expect)


def test_moments():
    x = synth.normal(0, 1, (1 << 20,), 1.0, "f64")
    assert abs(x.mean()) < 5e-3
    assert abs(x.var() - 1.0) < 5e-3
    # fourth moment of a normal is 3
    assert abs(np.mean(x ** 4) - 3.0) < 0.05


def test_decay_schedule():
    lam = synth.decay_schedule(16)
    assert lam.dtype == np.float32
    for h in range(16):
        assert lam[h] == np.float32(math.exp(-2.0 ** (-8.0 * (h + 1) / 16)))
    assert np.all(np.diff(lam) > 0)
    for H in (32, 64):
        lh = synth.decay_schedule(H)
        assert 0.39 < lh.min() and lh.max() < 0.9962
