"""Pins for the seeded input generator (CPU)."""
import math

import numpy as np
import pytest

from attention_forward_backward_amd import synth


def test_splitmix64_published_vectors():
    # Outputs of the sequential SplitMix64 generator as published with its
    # reference implementation: state 0, and state 1234567.
    assert synth.splitmix64_sequence(0, 3) == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert synth.splitmix64_sequence(1234567, 3) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_vectorised_mix_matches_scalar():
    kappa = synth.stream_key(7, 2)
    u1, u2 = synth.uniforms(7, 2, 100, 5)
    for n in range(5):
        i = 100 + n
        a = synth.mix64_int(kappa + (2 * i + 1) * synth.GOLDEN)
        b = synth.mix64_int(kappa + (2 * i + 2) * synth.GOLDEN)
        assert u1[n] == ((a >> 11) + 1) * 2.0 ** -53
        assert u2[n] == (b >> 11) * 2.0 ** -53


def test_index_addressable_and_deterministic():
    full = synth.normal_f32(3, 1, (4, 100))
    part = synth.normal_f32(3, 1, (50,), start=170)
    np.testing.assert_array_equal(full.reshape(-1)[170:220], part)
    np.testing.assert_array_equal(full, synth.normal_f32(3, 1, (4, 100)))
    assert not np.array_equal(full, synth.normal_f32(4, 1, (4, 100)))
    assert not np.array_equal(full, synth.normal_f32(3, 2, (4, 100)))


def test_box_muller_closed_form():
    # With u1 = exp(-1/2) and u2 = 0 the cosine branch gives exactly 1.
    assert math.sqrt(-2 * math.log(math.exp(-0.5))) * math.cos(0.0) == pytest.approx(1.0, abs=1e-15)
    u1, u2 = synth.uniforms(0, 0, 0, 8)
    z = synth.normal_f32(0, 0, (8,))
    ref = (np.sqrt(-2 * np.log(u1)) * np.cos(2 * math.pi * u2)).astype(np.float32)
    np.testing.assert_array_equal(z, ref)


def test_moments_and_sigma():
    x = synth.normal_f32(0, 3, (1 << 20,)).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.var() - 1.0) < 5e-3
    assert abs(np.mean(x ** 4) / x.var() ** 2 - 3.0) < 3e-2   # Gaussian kurtosis
    y = synth.normal_f32(0, 3, (1 << 20,), sigma=0.5).astype(np.float64)
    np.testing.assert_allclose(y, 0.5 * x, rtol=1e-6, atol=1e-7)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9,
                  -2.5, 3.0e38, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 2.9999e38, 1.0 + 2 ** -7],
                    dtype=np.float32)
    # ties (1 + 2^-8 and 1 + 3*2^-8) go to the even mantissa
    np.testing.assert_array_equal(got[:5], want[:5])
    assert got[6] == np.float32(1.0 + 2 ** -7)
    assert abs(got[5] - 3.0e38) / 3.0e38 < 2 ** -8


def test_bf16_inputs_exact_in_f32():
    inp = synth.make_inputs((1, 2, 9, 8), seed=1, dtype="bf16")
    for n in ("q", "k", "v", "do"):
        back = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(inp[n]))
        np.testing.assert_array_equal(back, inp[n])


def test_config_accounting():
    c = synth.CONFIGS["decoder_step"]
    assert c.pairs == 8 * 12 * 512 * 513 // 2 == 12607488
    assert c.flops["fwd_bwd"] == 14 * 64 * 12607488
    e = synth.CONFIGS["ragged_encoder"]
    assert e.pairs == 32 * 8 * 197 * 197 and not e.causal and e.sigma_qkv == 0.5


def test_key_lengths_range_and_determinism():
    a = synth.key_lengths(0, 4096, 64, 512)
    assert a.dtype == np.int32 and a.min() >= 64 and a.max() <= 512
    assert a.min() == 64 and a.max() == 512  # both ends reachable
    assert np.array_equal(a, synth.key_lengths(0, 4096, 64, 512))
    assert not np.array_equal(a, synth.key_lengths(1, 4096, 64, 512))
    assert np.array_equal(synth.key_lengths(3, 5, 7, 7), np.full(5, 7))


def test_cross_inputs_shapes_and_independent_keys():
    x = synth.cross_inputs((2, 3, 5, 32), (2, 3, 9, 32), 0, "bf16")
    assert x["q"].shape == x["do"].shape == (2, 3, 5, 32)
    assert x["k"].shape == x["v"].shape == (2, 3, 9, 32)
    assert set(x) >= {"q_bits", "k_bits", "v_bits", "do_bits"}
    same = synth.make_inputs((2, 3, 9, 32), 0, "f32")
    assert not np.array_equal(synth.cross_inputs((2, 3, 9, 32), (2, 3, 9, 32), 0)["k"], same["k"])
