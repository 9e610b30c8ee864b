"""GPU parity of the video decoder (fh_vae_decode) against the float64 oracle
(oracle/vae.py), every output element, at the toy, ragged and slice sizes
(the slice and ragged_h sizes run the halo-tiled convolution on their wide
layers, ragged_h on frames whose rows end mid-tile).

Bar: max |gpu - oracle| <= 4e-3 on the frames in [0, 1] (about one RGB24
level). Both sides round to F16 at the same points (the audio-cpp page's
storage rules); they differ in the sums, F32 on the device (relative error
about sqrt(K) 6e-8, K <= 27 x 256) against float64. That difference flips an
F16 rounding (half a step, 2.4e-4 relative) in a small share of the stored
values, each flip a change of one F16 step that later layers average; the
frames carry half a step of v's F16 rounding (2.4e-4 at |v| ~ 1) plus those
propagated flips. A wrong tap, channel order or padding rule moves outputs
by O(0.1).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import vae as V

pytestmark = pytest.mark.gpu
TOL_VAE = 4e-3


def say(msg):
    print(msg, flush=True)


def decode(fh, vc, z=None):
    W = synth.make_vae_weights(vc)
    vw = fh.fh_vae_weights_bind(vc, W)
    if z is None:
        z = synth.vae_latent(vc)
    out = fh.fh_vae_decode(vw, torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    return out, W, z, vw


@pytest.mark.parametrize("name", ["toy", "ragged", "latent8", "ragged_h", "slice"])
def test_decoder_against_oracle(fh, name):
    vc = synth.VAE_CONFIGS["toy"].replace(latent_ch=8) if name == "latent8" else synth.VAE_CONFIGS[name]
    say(f"decoder {name}: latent {vc.latent_ch}x{vc.frames}x{vc.height}x{vc.width}, widths {vc.widths}")
    out, W, z, _ = decode(fh, vc)
    got = out.cpu().numpy()
    want = V.decode(z, synth.vae_weights_f32(W), vc)
    err = np.abs(got - want)
    exact = V.decode(z, synth.vae_weights_f32(W), vc, half=False) if name != "slice" else None
    say(f"  max abs err {err.max():.3e}, mean {err.mean():.3e}, share > 1e-3 {np.mean(err > 1e-3):.2e}"
        + (f"; F16 oracle vs exact {np.abs(want - exact).max():.3e}" if exact is not None else ""))
    assert got.shape == want.shape == (3, vc.out_frames, vc.out_height, vc.out_width)
    assert np.all(np.isfinite(got)) and got.min() >= 0.0 and got.max() <= 1.0
    assert err.max() <= TOL_VAE


def test_decoder_deterministic_and_workspace_reuse(fh):
    """The same call twice gives the same bits, with the workspace holding the
    previous call's contents (every buffer is written before it is read)."""
    vc = synth.VAE_CONFIGS["ragged"]
    W = synth.make_vae_weights(vc)
    vw = fh.fh_vae_weights_bind(vc, W)
    ws = torch.full((fh.fh_vae_workspace_bytes(vc),), 255, dtype=torch.uint8, device="cuda")
    z = torch.from_numpy(synth.vae_latent(vc)).cuda()
    a = fh.fh_vae_decode(vw, z, workspace=ws).clone()
    b = fh.fh_vae_decode(vw, z, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decoded_frames_feed_the_colour_match(fh):
    """The decoder's planar frames are fh_color_match's input as they are."""
    vc = synth.VAE_CONFIGS["toy"]
    out, _, _, _ = decode(fh, vc)
    _, pic = synth.color_inputs(1, 4, 4, 128, 128)
    got = fh.fh_color_match(out, torch.from_numpy(pic).cuda(), 1.0)
    torch.cuda.synchronize()
    from oracle import color
    want = color.color_match(out.cpu().numpy().astype(np.float64), pic.astype(np.float64), 1.0)
    assert np.abs(got.cpu().numpy() - want).max() <= 2e-4
