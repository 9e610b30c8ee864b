"""Pins of the video-decoder oracle (oracle/vae.py) against things other than
itself: brute-force loops, torch's conv3d on explicitly padded input, closed
forms (delta and constant kernels), causality, index maps of depth to space
and of the patch unfold, IEEE half rounding. No GPU."""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import vae as V

rng = np.random.default_rng(77)


def _conv_loops(x, w, b):
    """The convolution of V1 written out element by element."""
    C, T, H, W = x.shape
    Co = w.shape[0]
    out = np.zeros((Co, T, H, W))
    for o, t, h, ww in itertools.product(range(Co), range(T), range(H), range(W)):
        s = b[o]
        for a, p, q, i in itertools.product(range(3), range(3), range(3), range(C)):
            tt, hh, w2 = max(t + a - 2, 0), h + p - 1, ww + q - 1     # frames before 0 repeat frame 0
            if 0 <= hh < H and 0 <= w2 < W:
                s += w[o, a, p, q, i] * x[i, tt, hh, w2]
        out[o, t, h, ww] = s
    return out


def test_conv3d_equals_brute_force_loops():
    x = rng.standard_normal((2, 3, 3, 4))
    w = rng.standard_normal((3, 3, 3, 3, 2))
    b = rng.standard_normal(3)
    np.testing.assert_allclose(V.conv3d(x, w, b, half=False), _conv_loops(x, w, b), atol=1e-12)


def test_conv3d_equals_torch_on_padded_input():
    """torch's conv3d (cross-correlation, weights [C_out, C_in, kt, kh, kw]) on the
    input padded by hand: two copies of frame 0 in front, zeros around in space."""
    x = rng.standard_normal((5, 4, 6, 7))
    w = rng.standard_normal((4, 3, 3, 3, 5))
    b = rng.standard_normal(4)
    xp = np.concatenate([x[:, :1], x[:, :1], x], axis=1)
    xp = np.pad(xp, ((0, 0), (0, 0), (1, 1), (1, 1)))
    ref = F.conv3d(torch.from_numpy(xp)[None], torch.from_numpy(np.moveaxis(w, 4, 1).copy()),
                   torch.from_numpy(b))[0].numpy()
    np.testing.assert_allclose(V.conv3d(x, w, b, half=False), ref, atol=1e-11)


def test_delta_kernel_is_the_identity_and_causal():
    """A kernel with 1 at the current frame's centre tap (time tap 2: the
    latest frame under causal padding) returns its input; a kernel at time
    tap 0 returns the input two frames back, frame 0 for the first two."""
    x = rng.standard_normal((3, 5, 4, 4))
    w = np.zeros((3, 3, 3, 3, 3))
    for i in range(3):
        w[i, 2, 1, 1, i] = 1.0
    np.testing.assert_array_equal(V.conv3d(x, w, np.zeros(3), half=False), x)
    w0 = np.zeros_like(w)
    for i in range(3):
        w0[i, 0, 1, 1, i] = 1.0
    back = V.conv3d(x, w0, np.zeros(3), half=False)
    np.testing.assert_array_equal(back[:, 2:], x[:, :3])
    np.testing.assert_array_equal(back[:, 0], x[:, 0])
    np.testing.assert_array_equal(back[:, 1], x[:, 0])


def test_constant_input_and_kernel():
    """Input c everywhere, every tap a: interior outputs are 27 C a c + b; an
    edge position loses the 9 taps of each missing row or column; time never
    loses taps (causal replicate)."""
    C, c, a = 4, 0.5, 0.25
    x = np.full((C, 3, 5, 6), c)
    w = np.full((2, 3, 3, 3, C), a)
    out = V.conv3d(x, w, np.array([1.0, -1.0]), half=False)
    np.testing.assert_allclose(out[0, :, 1:-1, 1:-1], 27 * C * a * c + 1.0)
    np.testing.assert_allclose(out[1, :, 0, 1:-1], 18 * C * a * c - 1.0)      # top row: 2 of 3 rows
    np.testing.assert_allclose(out[0, :, 0, 0], 12 * C * a * c + 1.0)         # corner: 2 x 2 of 3 x 3


def test_causality():
    """Changing frame t changes no output frame before t."""
    x = rng.standard_normal((2, 6, 3, 3))
    w = rng.standard_normal((2, 3, 3, 3, 2))
    y0 = V.conv3d(x, w, np.zeros(2), half=False)
    x2 = x.copy()
    x2[:, 4] += 1.0
    y1 = V.conv3d(x2, w, np.zeros(2), half=False)
    np.testing.assert_array_equal(y1[:, :4], y0[:, :4])
    assert np.abs(y1[:, 4:] - y0[:, 4:]).max() > 0.1


def test_depth_to_space_index_map():
    """Output channel s C' + c, s = 4 dt + 2 dh + dw, of the up-sampling
    convolution lands at (2t + dt - 1, 2h + dh, 2w + dw) of channel c (frame
    2t + dt = 0 dropped); checked with a delta kernel carrying the index."""
    Cp, T, H, W = 2, 3, 2, 3
    x = rng.standard_normal((Cp, T, H, W))
    w = np.zeros((8 * Cp, 3, 3, 3, Cp))
    for s, c in itertools.product(range(8), range(Cp)):
        w[s * Cp + c, 2, 1, 1, c] = 1.0 + s                # identity scaled by 1 + s
    z = V.upsample(x, w, np.zeros(8 * Cp), half=False)
    assert z.shape == (Cp, 2 * T - 1, 2 * H, 2 * W)
    for c, t, dt, h, dh, ww, dw in itertools.product(range(Cp), range(T), range(2), range(H), range(2), range(W),
                                                     range(2)):
        if 2 * t + dt == 0:
            continue
        s = 4 * dt + 2 * dh + dw
        assert z[c, 2 * t + dt - 1, 2 * h + dh, 2 * ww + dw] == (1.0 + s) * x[c, t, h, ww]


def test_unpatchify_index_map():
    P, T, H, W = 4, 2, 3, 2
    y = rng.standard_normal((3 * P * P, T, H, W))
    out = V.unpatchify(y, 3, P)
    assert out.shape == (3, T, H * P, W * P)
    for c, ph, pw, t, h, w in itertools.product(range(3), range(P), range(P), range(T), range(H), range(W)):
        assert out[c, t, h * P + ph, w * P + pw] == y[c * P * P + ph * P + pw, t, h, w]


def test_norm_silu_matches_torch():
    x = rng.standard_normal((6, 2, 3, 4))
    g = 1.0 + 0.1 * rng.standard_normal(6)
    xt = torch.from_numpy(np.moveaxis(x, 0, -1).copy())
    ref = F.silu(F.rms_norm(xt, (6,), torch.from_numpy(g), eps=1e-6))
    np.testing.assert_allclose(V.norm_silu(x, g, 1e-6, half=False), np.moveaxis(ref.numpy(), -1, 0), atol=1e-13)


def test_half_rounding_is_ieee_binary16():
    """f16 rounds as torch's float16 cast (round to nearest even), including
    halfway cases and the subnormal range."""
    v = np.concatenate([rng.standard_normal(1000) * 10, rng.standard_normal(100) * 1e-6,
                        1.0 + np.arange(8) * 2.0 ** -11, [65504.0, 2.0 ** -24, 3 * 2.0 ** -25]])
    ref = torch.from_numpy(v).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(V.f16(v), ref)
    assert V.f16(1.0 + 2.0 ** -11) == 1.0 and V.f16(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9   # ties to even


def test_half_storage_points():
    """With half storage a convolution's output is the F16 rounding of (the F16
    rounding of its exact sum) + bias; without it the exact value."""
    x = rng.standard_normal((3, 2, 3, 3))
    w = synth.f16_to_f32(synth.f16_bits(rng.standard_normal((2, 3, 3, 3, 3)) * 0.2)).astype(np.float64)
    b = np.array([0.37, -1.1])
    exact = V.conv3d(V.f16(x), w, np.zeros(2), half=False)
    np.testing.assert_array_equal(V.conv3d(x, w, b, half=True), V.f16(V.f16(exact) + b[:, None, None, None]))


def test_decode_shapes_range_and_half_vs_exact():
    """The toy decoder: 2 latent frames of 4 x 4 -> 9 frames of 128 x 128 in
    [0, 1]; F16 storage moves it by a few half-precision steps at most."""
    vc = synth.VAE_CONFIGS["toy"]
    W = synth.vae_weights_f32(synth.make_vae_weights(vc))
    z = synth.vae_latent(vc)
    out = V.decode(z, W, vc)
    assert out.shape == (3, vc.out_frames, vc.out_height, vc.out_width) == (3, 9, 128, 128)
    assert out.min() >= 0.0 and out.max() <= 1.0 and 0.05 < out.std() < 0.5
    exact = V.decode(z, W, vc, half=False)
    assert 1e-5 < np.abs(out - exact).max() < 2e-2


def test_slice_decoder_sizes():
    """5 latent frames of 16 x 16 decode to 33 frames of 512 x 512 (the gizai
    page's 33 frames; stride 8 in time, 32 in space)."""
    vc = synth.VAE_CONFIGS["slice"]
    assert (vc.out_frames, vc.out_height, vc.out_width) == (33, 512, 512)
    specs = synth.vae_param_specs(vc)
    assert specs[-2][1] == (48, 3, 3, 3, 32) and dict((n, s) for n, s, _ in specs)["up2.up.w"] == (256, 3, 3, 3, 64)
