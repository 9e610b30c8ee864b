"""Pins of the colour-correction oracle (oracle/color.py) against the colour
standards it restates and against the invariants of the statistics match:
BT.709's luminance coefficients and the D65 white in XYZ, CIELAB's white and
grey axis, the Lab coordinates of the sRGB primaries, exact round trips, the
matched statistics, the strength's end points, and a brute-force scalar loop."""
import math

import numpy as np
import pytest

from oracle import color as C


def test_rgb_to_xyz_matrix_has_bt709_luminance_and_d65_white():
    np.testing.assert_allclose(C.RGB_TO_XYZ[1], [0.2126, 0.7152, 0.0722], atol=5e-5)   # BT.709 luma row
    np.testing.assert_allclose(C.RGB_TO_XYZ @ np.ones(3), C.WHITE, rtol=0, atol=1e-15)
    # D65 from the sRGB standard's chromaticity; CIE's tabulated white is within 3e-4
    np.testing.assert_allclose(C.WHITE, [0.95047, 1.0, 1.08883], atol=3e-4)


def test_white_black_and_greys_lie_on_the_l_axis():
    np.testing.assert_allclose(C.rgb_to_lab(np.ones(3)), [100.0, 0.0, 0.0], atol=1e-12)
    np.testing.assert_allclose(C.rgb_to_lab(np.zeros(3)), [0.0, 0.0, 0.0], atol=1e-12)
    g = np.linspace(0, 1, 33)[:, None].repeat(3, axis=1)
    lab = C.rgb_to_lab(g)
    np.testing.assert_allclose(lab[:, 1:], 0.0, atol=1e-12)
    assert np.all(np.diff(lab[:, 0]) > 0)
    # mid grey: linear 0.21404, L = 116 cbrt(0.21404) - 16
    want = 116.0 * math.pow(((0.5 + 0.055) / 1.055) ** 2.4, 1.0 / 3.0) - 16.0
    assert abs(lab[16, 0] - want) < 1e-12 and abs(want - 53.389) < 1e-3


@pytest.mark.parametrize("rgb,lab", [
    ((1, 0, 0), (53.2408, 80.0925, 67.2032)),
    ((0, 1, 0), (87.7347, -86.1827, 83.1793)),
    ((0, 0, 1), (32.2970, 79.1875, -107.8602)),
])
def test_lab_of_the_srgb_primaries(rgb, lab):
    """The commonly published coordinates (CIE's tabulated D65 white): the
    white-point convention (reading C6) moves them by under 1e-2."""
    np.testing.assert_allclose(C.rgb_to_lab(np.array(rgb, float)), lab, atol=1e-2)


def test_transfer_curve_and_lab_round_trips():
    x = np.linspace(0, 1, 1001)
    np.testing.assert_allclose(C.linear_to_srgb(C.srgb_to_linear(x)), x, atol=1e-12)
    rng = np.random.default_rng(0)
    rgb = rng.random((500, 3))
    np.testing.assert_allclose(C.lab_to_rgb(C.rgb_to_lab(rgb)), rgb, atol=1e-12)
    # the two pieces of each curve meet at the breakpoints (to the standard's rounding)
    assert abs(0.04045 / 12.92 - ((0.04045 + 0.055) / 1.055) ** 2.4) < 1e-6
    assert abs(C._f(np.array(C._DELTA ** 3)) - C._DELTA) < 1e-15


def test_matching_moves_the_statistics_to_the_picture():
    rng = np.random.default_rng(1)
    lab = rng.normal([50, 10, -5], [12, 5, 8], (4000, 3))
    mu, sd = C.lab_stats(lab)
    mu_ref, sd_ref = np.array([60.0, -3.0, 7.0]), np.array([9.0, 4.0, 11.0])
    out = C.match_lab(lab, mu, sd, mu_ref, sd_ref, 1.0)
    m2, s2 = C.lab_stats(out)
    np.testing.assert_allclose(m2, mu_ref, atol=1e-10)
    np.testing.assert_allclose(s2, sd_ref, atol=1e-10)
    np.testing.assert_array_equal(C.match_lab(lab, mu, sd, mu_ref, sd_ref, 0.0), lab)
    half = C.match_lab(lab, mu, sd, mu_ref, sd_ref, 0.5)
    np.testing.assert_allclose(half, 0.5 * (lab + out), atol=1e-12)


def test_flat_frame_takes_the_picture_mean():
    lab = np.tile([[40.0, 2.0, 3.0]], (16, 1))
    out = C.match_lab(lab, *C.lab_stats(lab), np.array([55.0, -1.0, 4.0]), np.array([5.0, 6.0, 7.0]), 1.0)
    np.testing.assert_allclose(out, np.tile([[55.0, -1.0, 4.0]], (16, 1)), atol=1e-12)


def test_flat_frame_in_color_match_takes_the_picture_mean_colour():
    """A frame of one colour has deviation 0 in every channel (C3): it becomes
    the picture's mean Lab colour, whatever residue summation leaves."""
    rng = np.random.default_rng(4)
    pic = rng.uniform(0.2, 0.8, (3, 9, 7))
    frames = np.broadcast_to(np.array([0.3, 0.6, 0.2])[:, None, None, None], (3, 2, 16, 12)).copy()
    out = C.color_match(frames, pic, 1.0)
    mu_ref = C.rgb_to_lab(np.moveaxis(pic, 0, -1)).reshape(-1, 3).mean(axis=0)
    np.testing.assert_allclose(C.rgb_to_lab(np.moveaxis(out, 0, -1)).reshape(-1, 3), np.tile(mu_ref, (2 * 16 * 12, 1)),
                               atol=1e-9)


def test_grey_frame_takes_the_picture_chroma():
    """C7: on a grey frame (R = G = B, greys varying) a* and b* hold only
    rounding noise; they count as flat and take the picture's mean chroma,
    while L* is matched as usual. Without the threshold sd_ref / sd amplifies
    the noise into arbitrary chroma."""
    rng = np.random.default_rng(5)
    pic = rng.uniform(0.2, 0.8, (3, 9, 7))
    g = rng.uniform(0.1, 0.9, (1, 2, 16, 12))
    frames = np.repeat(g, 3, axis=0)
    out = C.color_match(frames, pic, 1.0)
    ref = C.rgb_to_lab(np.moveaxis(pic, 0, -1)).reshape(-1, 3)
    for f in range(2):
        lab = C.rgb_to_lab(np.moveaxis(out[:, f], 0, -1)).reshape(-1, 3)
        clipped = np.any((out[:, f] <= 0) | (out[:, f] >= 1), axis=0).reshape(-1)
        np.testing.assert_allclose(lab[~clipped, 1:], np.tile(ref.mean(axis=0)[1:], ((~clipped).sum(), 1)),
                                   atol=1e-6)
        src = C.rgb_to_lab(np.moveaxis(frames[:, f], 0, -1)).reshape(-1, 3)
        assert np.abs(src[:, 1:]).max() < 1e-9 and src[:, 0].std() > 1.0   # grey in, real L* spread
    # the decision sits far from the noise on either side
    sd = C.lab_stats(C.rgb_to_lab(np.moveaxis(frames[:, 0], 0, -1)))[1]
    assert sd[1] < 1e-9 < C.FLAT_SD < 1.0 < sd[0]


def test_zero_strength_returns_the_frames():
    rng = np.random.default_rng(2)
    frames, pic = rng.random((3, 2, 5, 6)), rng.random((3, 7, 4))
    np.testing.assert_allclose(C.color_match(frames, pic, 0.0), frames, atol=1e-12)


def _lab_scalar(r, g, b):
    lin = [c / 12.92 if c <= 0.04045 else ((c + 0.055) / 1.055) ** 2.4 for c in (r, g, b)]
    xyz = [sum(C.RGB_TO_XYZ[i][j] * lin[j] for j in range(3)) / C.WHITE[i] for i in range(3)]
    d = 6.0 / 29.0
    f = [t ** (1.0 / 3.0) if t > d ** 3 else t / (3 * d * d) + 4.0 / 29.0 for t in xyz]
    return [116 * f[1] - 16, 500 * (f[0] - f[1]), 200 * (f[1] - f[2])]


def _rgb_scalar(L, a, b):
    d = 6.0 / 29.0
    fy = (L + 16) / 116
    fs = [fy + a / 500, fy, fy - b / 200]
    xyz = [C.WHITE[i] * (t ** 3 if t > d else 3 * d * d * (t - 4.0 / 29.0)) for i, t in enumerate(fs)]
    lin = [sum(C.XYZ_TO_RGB[i][j] * xyz[j] for j in range(3)) for i in range(3)]
    out = [12.92 * c if c <= 0.0031308 else 1.055 * max(c, 0.0) ** (1 / 2.4) - 0.055 for c in lin]
    return [min(max(c, 0.0), 1.0) for c in out]


def test_color_match_equals_a_scalar_loop():
    rng = np.random.default_rng(3)
    frames, pic, s = rng.random((3, 2, 3, 4)), rng.random((3, 5, 3)), 0.7   # RGB planes
    ref = [_lab_scalar(pic[0, y, x], pic[1, y, x], pic[2, y, x]) for y in range(5) for x in range(3)]
    n = len(ref)
    mr = [sum(v[c] for v in ref) / n for c in range(3)]
    sr = [math.sqrt(sum((v[c] - mr[c]) ** 2 for v in ref) / n) for c in range(3)]
    want = np.empty_like(frames)
    for f in range(frames.shape[1]):
        lab = [_lab_scalar(frames[0, f, y, x], frames[1, f, y, x], frames[2, f, y, x])
               for y in range(3) for x in range(4)]
        m = [sum(v[c] for v in lab) / len(lab) for c in range(3)]
        sd = [math.sqrt(sum((v[c] - m[c]) ** 2 for v in lab) / len(lab)) for c in range(3)]
        outs = []
        for v in lab:
            w = [v[c] + s * (mr[c] + (v[c] - m[c]) * sr[c] / sd[c] - v[c]) for c in range(3)]
            outs.append(_rgb_scalar(*w))
        want[:, f] = np.array(outs).T.reshape(3, 3, 4)
    np.testing.assert_allclose(C.color_match(frames, pic, s), want, atol=1e-12)


def test_dark_colours_use_cielabs_linear_branch():
    """Below Y = (6/29)^3 CIE's L* is kappa Y with kappa = 24389 / 27 (and a*, b*
    follow the same linear form): dark greys pin that branch."""
    for c in (0.0, 0.004, 0.01, 0.02):
        y = c / 12.92                                # below the sRGB breakpoint: linear
        assert y < (6 / 29) ** 3
        np.testing.assert_allclose(C.rgb_to_lab(np.full(3, c)), [24389 / 27 * y, 0.0, 0.0], atol=1e-12)
