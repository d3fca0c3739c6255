"""The seeded input recipe: deterministic, right shapes, encodings as stated."""
import numpy as np

from decoder_only_transformer_decode_amd import synth


def test_weights_deterministic_and_shaped():
    s = synth.tiny_shape(wfmt=synth.W_Q8_0)
    a = synth.gen_weights(s, 7, threads=3)
    b = synth.gen_weights(s, 7, threads=1)
    shapes = synth.matrix_shapes(s)
    for name, parts in a.items():
        for k, v in parts.items():
            assert np.array_equal(v, b[name][k])
        if name in shapes:
            r, c = shapes[name]
            assert parts["q"].shape == (r, c) and parts["s"].shape == (r, c // 32)
    assert set(a) == set(synth.tensor_order(s))


def test_streams_differ_between_tensors_and_seeds():
    s = synth.tiny_shape()
    a = synth.gen_weights(s, 1)
    b = synth.gen_weights(s, 2)
    assert not np.array_equal(a["L0.wq"]["q"], b["L0.wq"]["q"])
    assert not np.array_equal(a["L0.wq"]["q"][:8], a["L0.wk"]["q"][:8])


def test_bf16_encoding_round_trip():
    x = np.array([1.0, -2.5, 3.0e-3, 1.00390625, 1.01171875], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    y = synth.bf16_bits_to_f32(b)
    assert y[0] == 1.0 and y[1] == -2.5
    assert y[3] == 1.0           # tie 1 + 2^-8 rounds to even (1.0)
    assert y[4] == 1.015625      # tie 1 + 3*2^-8 rounds to even (1 + 2^-6)


def test_prompts_and_contexts_in_range():
    t = synth.prompt_tokens(128256, 512)
    assert t.min() >= 0 and t.max() < 128256 and t.dtype == np.int32
    c = synth.context_lengths(64)
    assert c.min() >= 512 and c.max() <= 4096 and len(c) == 64
