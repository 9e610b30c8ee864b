"""Float64 oracle of the colour correction after the VAE decode (decoded frames
matched to the reference picture in CIELAB).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: the gizai:flashhead reference page (overview paragraph)
has the decoded frames' colours matched to the picture's through Lab means
and deviations; the SoulX-FlashHead audio-cpp page (request options) names a
correction strength, 1 by default, 0 disabling it, and (variant boundaries)
keeps colour processing in F32. Colour science is fixed by its standards:
sRGB's transfer curve and BT.709 primaries with the D65 white (IEC 61966-2-1),
CIELAB (CIE 15) relative to that white.

READINGS (the plainest ones the rest supports):
  C1 frames and picture are sRGB values in [0, 1] held as RGB planes: the
     picture [3, H, W] as the gizai:flashhead page's FlashHead.picture makes
     it, the decoded frames [3, F, H, W] (channels first, as a video VAE
     emits them);
  C2 the statistics are per frame and per Lab channel: mean and standard
     deviation (population) over the frame's pixels, and the same over the
     picture;
  C3 matching moves each channel to the picture's statistics,
     v' = mu_ref + (v - mu) * sd_ref / sd   (v' = mu_ref where sd = 0, C7);
  C4 the strength s blends in Lab: v'' = v + s (v' - v) (s = 0 leaves the
     frame as it was, s = 1 is the full match);
  C5 back to sRGB through the inverse transforms, clamped to [0, 1];
  C6 one white for both the RGB -> XYZ matrix and the Lab reference: D65 at
     the chromaticity the sRGB standard gives (0.3127, 0.3290), so sRGB white
     is exactly L* = 100, a* = b* = 0 (CIE's tabulated D65 differs in the
     fourth decimal of X and Z, which moves Lab values by under 0.01);
  C7 a channel whose deviation is below FLAT_SD = 1e-3 Lab units counts as
     flat (C3's sd = 0 rule): on a grey frame (R = G = B) a* and b* carry only
     rounding noise (about 1e-14 here, 1e-5 in float32), which sd_ref / sd
     would blow up into arbitrary chroma; a thousandth of a Lab unit is far
     below anything visible (one RGB24 level is about 0.4 L* units).
"""
from __future__ import annotations

import numpy as np

__all__ = ["FLAT_SD", "RGB_TO_XYZ", "WHITE", "srgb_to_linear", "linear_to_srgb", "rgb_to_lab", "lab_to_rgb",
           "lab_stats", "match_lab", "color_match"]

# C7: deviations below this (Lab units) count as a flat channel
FLAT_SD = 1e-3

# BT.709 primaries and the D65 white point (xy chromaticities)
_PRIMARIES = np.array([[0.64, 0.33], [0.30, 0.60], [0.15, 0.06]])
_D65 = np.array([0.3127, 0.3290])


def _xyz(xy):
    """XYZ of chromaticity (x, y) at Y = 1."""
    x, y = xy
    return np.array([x / y, 1.0, (1.0 - x - y) / y])


def _rgb_to_xyz_matrix():
    """The matrix whose columns are the primaries' XYZ, scaled so that
    R = G = B = 1 gives the white point's XYZ (Y = 1)."""
    P = np.stack([_xyz(p) for p in _PRIMARIES], axis=1)
    scale = np.linalg.solve(P, _xyz(_D65))
    return P * scale[None, :]


RGB_TO_XYZ = _rgb_to_xyz_matrix()
XYZ_TO_RGB = np.linalg.inv(RGB_TO_XYZ)
WHITE = _xyz(_D65)                      # Xn, Yn (= 1), Zn
_DELTA = 6.0 / 29.0


def srgb_to_linear(c):
    """sRGB transfer curve, inverse: linear below 0.04045, else a 2.4 power."""
    c = np.asarray(c, dtype=np.float64)
    return np.where(c <= 0.04045, c / 12.92, ((c + 0.055) / 1.055) ** 2.4)


def linear_to_srgb(c):
    c = np.asarray(c, dtype=np.float64)
    return np.where(c <= 0.0031308, 12.92 * c, 1.055 * np.maximum(c, 0.0) ** (1.0 / 2.4) - 0.055)


def _f(t):
    return np.where(t > _DELTA ** 3, np.cbrt(t), t / (3.0 * _DELTA ** 2) + 4.0 / 29.0)


def _finv(t):
    return np.where(t > _DELTA, t ** 3, 3.0 * _DELTA ** 2 * (t - 4.0 / 29.0))


def rgb_to_lab(rgb):
    """[..., 3] sRGB -> [..., 3] CIELAB (L*, a*, b*) relative to D65."""
    xyz = srgb_to_linear(rgb) @ RGB_TO_XYZ.T
    fx, fy, fz = (_f(xyz[..., i] / WHITE[i]) for i in range(3))
    return np.stack([116.0 * fy - 16.0, 500.0 * (fx - fy), 200.0 * (fy - fz)], axis=-1)


def lab_to_rgb(lab):
    """[..., 3] CIELAB -> [..., 3] sRGB, not clamped."""
    lab = np.asarray(lab, dtype=np.float64)
    fy = (lab[..., 0] + 16.0) / 116.0
    fx, fz = fy + lab[..., 1] / 500.0, fy - lab[..., 2] / 200.0
    xyz = np.stack([WHITE[0] * _finv(fx), WHITE[1] * _finv(fy), WHITE[2] * _finv(fz)], axis=-1)
    return linear_to_srgb(xyz @ XYZ_TO_RGB.T)


def lab_stats(lab):
    """Per-channel mean and population standard deviation over all pixels of
    [..., 3]. A channel whose values are all equal has deviation exactly 0
    (floating-point summation could leave a residue of ~1e-14 that C3's
    division would blow up)."""
    v = lab.reshape(-1, 3)
    flat = np.ptp(v, axis=0) == 0
    return np.where(flat, v[0], v.mean(axis=0)), np.where(flat, 0.0, v.std(axis=0))


def match_lab(lab, mu, sd, mu_ref, sd_ref, strength):
    """C3 and C4 on one frame's Lab values (C7: a channel with sd below FLAT_SD
    is flat and takes mu_ref)."""
    scale = np.divide(sd_ref, sd, out=np.zeros(3), where=sd >= FLAT_SD)
    matched = mu_ref + (lab - mu) * scale
    return lab + strength * (matched - lab)


def color_match(frames, picture, strength=1.0):
    """Frames [3, F, H, W] matched to picture [3, H', W'] (C1-C5), float64."""
    ref = rgb_to_lab(np.moveaxis(np.asarray(picture, dtype=np.float64), 0, -1))
    mu_ref, sd_ref = lab_stats(ref)
    fr = np.moveaxis(np.asarray(frames, dtype=np.float64), 0, -1)      # [F, H, W, 3]
    out = np.empty(fr.shape, dtype=np.float64)
    for i in range(fr.shape[0]):
        lab = rgb_to_lab(fr[i])
        mu, sd = lab_stats(lab)
        out[i] = np.clip(lab_to_rgb(match_lab(lab, mu, sd, mu_ref, sd_ref, strength)), 0.0, 1.0)
    return np.moveaxis(out, -1, 0)
