"""Checks of the seeded input generators (no forward-pass arithmetic)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_known_values():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0, 3.0e38], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(a)
    # 1+2^-8 is an exact tie -> even (down); 1+3*2^-8 ties -> even (up)
    assert [hex(int(b)) for b in bits[:6]] == ["0x3f80", "0x3f80", "0x3f82", "0xc020", "0x0", "0x8000"]
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bits[:6]), [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0, -0.0])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_weights_seeded_and_shaped():
    s = synth.small_shape(dtype=synth.BF16)
    w1 = synth.make_weights(s, 3)
    w2 = synth.make_weights(s, 3)
    np.testing.assert_array_equal(w1["embed"], w2["embed"])
    assert w1["embed"].shape == (s.vocab, s.hidden)
    for k, shp in s.layer_shapes().items():
        assert w1["layers"][1][k].shape == shp
    # bf16 models hold bf16-representable values
    e = w1["layers"][0]["wq"]
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(e)), e)
    assert abs(float(np.std(w1["embed"])) - 0.02) < 0.005
    assert abs(float(np.mean(w1["final_norm"])) - 1.0) < 0.1


def test_workloads():
    w = synth.workload("tiny_fp32")
    assert w.batch == 1 and len(w.prompts[0]) == 16 and w.decode_steps == 16
    w = synth.workload("decode_0p6b_bs64")
    lens = [len(p) for p in w.prompts]
    assert len(lens) == 64 and min(lens) >= 256 and max(lens) <= 4096
    assert w.max_ctx <= 4096 + 128
    for p in w.prompts:
        assert p.dtype == np.int32 and p.min() >= 0 and p.max() < synth.QWEN3_0P6B.vocab
    w = synth.workload("prefill_0p6b_4x4096")
    assert w.batch == 4 and all(len(p) == 4096 for p in w.prompts)
