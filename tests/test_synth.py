"""Pins of the seeded input generator against its published definitions."""
import numpy as np

import synth
from synth.weights import host_weights, prompt
from synth.workloads import TINY


def test_splitmix64_published_vector():
    # SplitMix64 reference stream for seed 1234567 (Steele, Lea & Flood 2014;
    # the widely reproduced test vector of the reference C implementation).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [synth.splitmix64_at(1234567, i) for i in range(5)] == want


def test_bf16_round_to_nearest_even():
    # bf16 keeps the top 16 bits of fp32; halfway cases go to the even mantissa.
    assert synth.f32_to_bf16(1.0) == 0x3F80
    assert synth.f32_to_bf16(1.0 + 2 ** -8) == 0x3F80          # tie -> even (down)
    assert synth.f32_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert synth.f32_to_bf16(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81  # above the tie
    assert synth.f32_to_bf16(-2.0) == 0xC000
    assert synth.f32_to_bf16(0.0) == 0x0000


def test_normal_statistics_and_offsets():
    x = synth.bf16_to_f32(synth.normal_bf16(1 << 20, 12345, 1.0)).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    # fourth moment of a normal is 3
    assert abs((x ** 4).mean() - 3.0) < 0.05
    a = synth.normal_bf16(1000, 99, 0.02)
    b = np.concatenate([synth.normal_bf16(300, 99, 0.02), synth.normal_bf16(700, 99, 0.02, offset=300)])
    assert np.array_equal(a, b)
    f = synth.normal_bf16_f32(1000, 99, 0.02)
    assert np.array_equal(f, synth.bf16_to_f32(a))


def test_tokens_in_range_and_spread():
    t = synth.tokens(100000, 7, 1024)
    assert t.min() >= 0 and t.max() < 1024
    counts = np.bincount(t, minlength=1024)
    assert counts.min() > 40 and counts.max() < 160


def test_weight_recipe_deterministic():
    w1 = host_weights(TINY)
    w2 = host_weights(TINY)
    assert np.array_equal(w1["layers"][1]["w_qkv"], w2["layers"][1]["w_qkv"])
    assert not np.array_equal(w1["layers"][0]["w_qkv"], w1["layers"][1]["w_qkv"])
    assert w1["layers"][0]["attn_norm"].dtype == np.float32
    assert np.all(w1["final_norm"] == 1.0)
    x = synth.bf16_to_f32(w1["layers"][0]["w_o"])
    assert abs(x.std() - 0.02) < 1e-3
    assert np.array_equal(prompt(TINY, 16), prompt(TINY, 16))
