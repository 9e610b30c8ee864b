"""GPU parity of the Lab colour match (fh_color_match) against the float64 oracle.

Bar: max |gpu - oracle| <= 2e-4 on sRGB values in [0, 1] (a twentieth of one
RGB24 level). Derivation: the device works in float32 (unit roundoff 6e-8);
Lab values up to 100 carry absolute errors of a few 1e-5 through the sRGB
power and the cube root, the transfer multiplies deviations by sd_ref / sd
(about 1 for these inputs), and the way back amplifies by at most the sRGB
curve's slope (12.92) times the XYZ -> RGB matrix's row sums (under 5):
about 1e-4 in the worst place, half the bar. Strength 0 must return the
frames bit for bit; the same call twice must give the same bits.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import color as C

pytestmark = pytest.mark.gpu
TOL_COLOR = 2e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def say(msg):
    print(msg, flush=True)


def run(fh, frames, pic, strength, out=None):
    o = fh.fh_color_match(dev(frames) if isinstance(frames, np.ndarray) else frames,
                          dev(pic) if isinstance(pic, np.ndarray) else pic, strength, out=out)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("shape", ["toy", "ragged", "slice"])
@pytest.mark.parametrize("strength", [1.0, 0.35, 1.5])
def test_color_match_against_oracle(fh, shape, strength):
    say(f"color_match {shape} {synth.COLOR_SHAPES[shape]} strength {strength}")
    fr, pic = synth.color_inputs(*synth.COLOR_SHAPES[shape])
    got = run(fh, fr, pic, strength).cpu().numpy()
    want = C.color_match(fr.astype(np.float64), pic.astype(np.float64), strength)
    err = np.abs(got - want).max()
    say(f"  max abs err {err:.3e}")
    assert got.shape == fr.shape and np.all((got >= 0) & (got <= 1))
    assert err <= TOL_COLOR


def test_strength_zero_is_the_frames_bit_for_bit(fh):
    fr, pic = synth.color_inputs(*synth.COLOR_SHAPES["toy"])
    F = dev(fr)
    got = run(fh, F, dev(pic), 0.0)
    assert torch.equal(got, F)
    same = run(fh, F, dev(pic), 0.0, out=F)           # in place: nothing changes
    assert same.data_ptr() == F.data_ptr() and torch.equal(F.cpu(), torch.from_numpy(fr))


def test_in_place_and_repeat_calls_give_the_same_bits(fh):
    fr, pic = synth.color_inputs(*synth.COLOR_SHAPES["toy"])
    P = dev(pic)
    a = run(fh, dev(fr), P, 0.8)
    b = run(fh, dev(fr), P, 0.8)
    F = dev(fr)
    c = run(fh, F, P, 0.8, out=F)
    assert torch.equal(a, b) and torch.equal(a, c)


def test_flat_black_and_one_pixel_picture(fh):
    """Degenerate statistics: a flat frame (sd = 0 in every channel) and an
    all-black frame take the picture's mean; a one-pixel picture (sd_ref = 0)
    makes every frame flat at that pixel's colour."""
    fr, pic = synth.color_inputs(4, 16, 12, 8, 8)
    fr[:, 1] = np.array([0.3, 0.6, 0.2], np.float32)[:, None, None]
    fr[:, 2] = 0.0
    for p, s in ((pic, 1.0), (pic, 0.6), (np.array([0.9, 0.1, 0.4], np.float32).reshape(3, 1, 1), 1.0)):
        got = run(fh, fr, p, s).cpu().numpy()
        want = C.color_match(fr.astype(np.float64), p.astype(np.float64), s)
        assert np.abs(got - want).max() <= TOL_COLOR
    got = run(fh, fr, np.array([0.9, 0.1, 0.4], np.float32).reshape(3, 1, 1), 1.0).cpu().numpy()
    np.testing.assert_allclose(got.reshape(3, -1), np.repeat([[0.9], [0.1], [0.4]], got[0].size, 1), atol=TOL_COLOR)


def test_grey_frames_take_the_picture_chroma(fh):
    """A grey frame's a* and b* deviations are rounding noise (~1e-5 in
    float32, ~1e-14 in the oracle): both sides treat them as flat (below 1e-3
    Lab units), so they agree to the bar instead of amplifying different noise."""
    fr, pic = synth.color_inputs(3, 16, 12, 8, 8)
    fr[1] = fr[0]
    fr[2] = fr[0]                               # R = G = B in every frame
    for s in (1.0, 0.5):
        got = run(fh, fr, pic, s).cpu().numpy()
        want = C.color_match(fr.astype(np.float64), pic.astype(np.float64), s)
        err = np.abs(got - want).max()
        say(f"  grey frames strength {s}: max abs err {err:.3e}")
        assert err <= TOL_COLOR


def test_scalar_path_on_misaligned_planes(fh):
    """Planes that start off a 16-byte boundary take the one-pixel path; it
    matches the oracle to the same bar."""
    fr, pic = synth.color_inputs(*synth.COLOR_SHAPES["toy"])
    buf = torch.zeros(fr.size + 1, device="cuda")
    view = buf[1:].view(fr.shape)
    view.copy_(dev(fr))
    out = torch.zeros(fr.size + 1, device="cuda")[1:].view(fr.shape)
    got = run(fh, view, dev(pic), 1.0, out=out).cpu().numpy()
    want = C.color_match(fr.astype(np.float64), pic.astype(np.float64), 1.0)
    assert np.abs(got - want).max() <= TOL_COLOR


def test_many_small_frames_and_empty_call(fh):
    """Many frames (a tall statistics grid) of a few pixels each; n_frames = 0
    does nothing."""
    fr, pic = synth.color_inputs(3000, 2, 3, 4, 4)
    got = run(fh, fr, pic, 1.0).cpu().numpy()
    want = C.color_match(fr.astype(np.float64), pic.astype(np.float64), 1.0)
    assert np.abs(got - want).max() <= TOL_COLOR
    empty = torch.zeros(3, 0, 4, 4, device="cuda")
    assert run(fh, empty, dev(pic), 1.0).shape == empty.shape
