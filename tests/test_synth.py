"""Host-side checks of the seeded synthetic generator (CPU only)."""
import numpy as np
import torch

from gru_corrected_draft_amd import synth


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30, -1e-30],
                                 np.float32)])
    ours = synth.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_block_seeded(monkeypatch):
    shp = synth.custom_shape(5000, 64, 32, 32, 32, "bf16", 99)
    a = synth.make_weights(shp)
    monkeypatch.setattr(synth, "BLOCK", 1 << 12)     # more blocks, other threading
    b = synth.make_weights(shp)
    # the block size is part of the recipe: same size -> identical, and the first
    # block's values agree because block 0 uses the same seed words.
    assert a.raw["fc2_w"].shape == (5000, 32)
    assert np.array_equal(a.raw["fc2_w"].reshape(-1)[:4096], b.raw["fc2_w"].reshape(-1)[:4096])
    c = synth.make_weights(shp)
    d = synth.make_weights(shp)
    assert all(np.array_equal(c.raw[k], d.raw[k]) for k in c.raw)


def test_weight_scales_follow_fan_in():
    shp = synth.custom_shape(20000, 256, 64, 128, 32, "fp32", 5)
    w = synth.make_weights(shp)
    for name, fan in [("lm_head", 256), ("embed", 64), ("gru_w_ih", 64), ("gru_w_hh", 128),
                      ("fc1_w", 128), ("fc2_w", 32), ("fc2_b", 32)]:
        std = float(np.std(w.f32(name)))
        assert abs(std * np.sqrt(fan) - 1.0) < 0.05, name


def test_inputs_shapes_and_ranges():
    shp = synth.MODELS["tiny"]
    inp = synth.make_inputs(shp, 3, 4096, 0)
    assert inp.hidden.shape == (3, 15, 256) and inp.hidden.dtype == np.float32
    assert inp.step_s.shape == (3, 14, 128) and inp.step_s.dtype == np.float32
    assert inp.verified.dtype == np.int32 and np.all((inp.verified >= 0) & (inp.verified < 4096))
    again = synth.make_inputs(shp, 3, 4096, 0)
    assert np.array_equal(inp.hidden, again.hidden) and np.array_equal(inp.verified, again.verified)
    other = synth.make_inputs(shp, 3, 4096, 1)
    assert not np.array_equal(inp.hidden, other.hidden)
