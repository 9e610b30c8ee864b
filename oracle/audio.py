"""Float64 oracle of the audio projection front end (speech states -> audio tokens).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: the gizai:flashhead reference page (overview paragraph)
takes, for each slice, the last 8 s of speech through wav2vec 2.0 base, keeps
its 12 layers' states at 200 frames, and makes 5 latent frames of 32 audio
tokens from 5 states around each of the slice's 33 frames; its type listing
(type FlashHead) names the layers proj1, proj1vf, proj2, proj3 (Linear) and
projNorm (tensors). Nothing else about this step is on the pages.

READINGS (the plainest ones the rest supports; every size is a parameter):
  A1 states S [L, T, C] per lane: L layers, T frames over the window at the
     video rate (200 frames = 8 s at 25 frames per second), C channels
     (768 for wav2vec 2.0 base);
  A2 the slice's V video frames are the window's last V frames: frame f sits
     at state frame T - V + f;
  A3 a frame's five states are those at offsets -2 .. +2 from it, clamped to [0, T - 1];
     a frame's feature is those states flattened in (offset, layer, channel)
     order, width 5 L C;
  A4 latent frames follow the video VAE's temporal stride s (8 for LTX):
     latent frame 0 is video frame 0, latent frame i >= 1 is video frames
     s(i-1)+1 .. s i (33 = 1 + 4 x 8), and its feature is the mean of its
     frames' features;
  A5 proj1 maps latent frame 0's feature and proj1vf the others' (both
     width 5 L C -> P), then SiLU; proj2 (P -> P), SiLU; proj3 (P -> tokens
     x D) gives the latent frame's tokens in order; projNorm is a LayerNorm
     over D with gain and bias (eps as the DiT's);
  A6 tokens are ordered latent frame by latent frame, as the DiT's
     frame-local cross-attention reads them.
Because proj1vf is linear and the activation follows it, projecting each of a
latent frame's video frames and averaging equals projecting the averaged
feature (pinned in tests).
"""
from __future__ import annotations

import numpy as np

from .dit import layer_norm, linear, silu, to64

__all__ = ["frame_states", "frame_features", "latent_features", "audio_project"]


def frame_states(T, V, window):
    """State frame indices [V, window] of each video frame's window (A2, A3)."""
    half = window // 2
    t = (T - V) + np.arange(V)[:, None] + np.arange(-half, window - half)[None, :]
    return np.clip(t, 0, T - 1)


def frame_features(states, V, window):
    """states [L, T, C] -> features [V, window * L * C] in (offset, layer, channel) order."""
    S = to64(states)
    L, T, C = S.shape
    idx = frame_states(T, V, window)                       # [V, window]
    win = S[:, idx, :]                                     # [L, V, window, C]
    return np.transpose(win, (1, 2, 0, 3)).reshape(V, window * L * C)


def latent_groups(V, stride):
    """Video frames of each latent frame (A4): [0], [1..s], [s+1..2s], ..."""
    if (V - 1) % stride:
        raise ValueError("video frames must be 1 + a multiple of the temporal stride")
    return [[0]] + [list(range(stride * (i - 1) + 1, stride * i + 1)) for i in range(1, 1 + (V - 1) // stride)]


def latent_features(feat, stride):
    """[V, F] -> [1 + (V-1)/stride, F]: frame 0, then the mean of each group of frames."""
    return np.stack([feat[g].mean(axis=0) for g in latent_groups(feat.shape[0], stride)])


def audio_project(states, Wa, acfg):
    """Audio tokens [B, La, D] of speech states [B, L, T, C] (A1-A6), one lane at a time."""
    out = []
    for s in np.asarray(states):
        X = latent_features(frame_features(s, acfg.video_frames, acfg.window), acfg.temporal_stride)
        h0 = silu(linear(X[:1], Wa["proj1.w"], Wa["proj1.b"]))
        h1 = silu(linear(X[1:], Wa["proj1vf.w"], Wa["proj1vf.b"]))
        h = silu(linear(np.concatenate([h0, h1]), Wa["proj2.w"], Wa["proj2.b"]))
        y = linear(h, Wa["proj3.w"], Wa["proj3.b"]).reshape(-1, acfg.dim)   # latent frame i -> rows i*T .. i*T+T-1
        out.append(layer_norm(y, acfg.eps, Wa["projNorm.g"], Wa["projNorm.b"]))
    return np.stack(out)
