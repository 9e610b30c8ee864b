"""The seeded data generator: bf16 rounding, determinism, lane seeds."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.0, -0.0, 3.0e-39, 65504.0]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_bits(x), ref)
    back = synth.bf16_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .to(torch.float32).numpy())


def test_weights_deterministic_and_subsettable():
    cfg = synth.CONFIGS["toy"]
    a = synth.make_weights(cfg)
    b = synth.make_weights(cfg, blocks=[1])
    assert synth.weights_digest(a) == synth.weights_digest(synth.make_weights(cfg))
    for k, v in b.items():
        np.testing.assert_array_equal(a[k], v)
    assert a["blocks.0.qkv.w"].dtype == np.uint16 and a["blocks.0.qkv.w"].shape == (768, 256)
    g = a["blocks.0.norm_q.g"]
    assert g.dtype == np.float32 and abs(g.mean() - 1) < 0.01


def test_lane_seeds():
    cfg = synth.CONFIGS["toy"]
    l3, m3, a3 = synth.slice_inputs(cfg, 3)
    l1, m1, a1 = synth.slice_inputs(cfg, 1)
    np.testing.assert_array_equal(l3[:1], l1)
    assert l3.shape == (3, 16, 2, 8, 8) and m3.shape == (3, 16, 1, 8, 8) and a3.shape == (3, 64, 256)
    assert not np.array_equal(l3[0], l3[1])
