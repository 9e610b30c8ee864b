"""Pins of the audio projection oracle (oracle/audio.py) against brute-force
loops, torch's library layers and its own structural readings: window indices
and clamping, feature order, the latent grouping, that averaging the frames'
features before the (linear) first layer equals averaging their projections,
token order, and the final LayerNorm's moments."""
import numpy as np
import pytest
import torch

import synth
from oracle import audio as A


def loop_features(S, V, window):
    """Explicit loops: feature[f][(d, l, c)] = S[l][clamp(T - V + f + d - 2)][c]."""
    L, T, C = S.shape
    out = np.zeros((V, window * L * C))
    for f in range(V):
        k = 0
        for d in range(window):
            t = min(max(T - V + f + d - window // 2, 0), T - 1)
            for l in range(L):
                for c in range(C):
                    out[f, k] = S[l, t, c]
                    k += 1
    return out


def test_window_indices_and_clamping():
    idx = A.frame_states(T=10, V=4, window=5)
    assert idx.tolist() == [[4, 5, 6, 7, 8], [5, 6, 7, 8, 9], [6, 7, 8, 9, 9], [7, 8, 9, 9, 9]]
    idx = A.frame_states(T=3, V=3, window=5)           # the window reaches below the first state
    assert idx.tolist() == [[0, 0, 0, 1, 2], [0, 0, 1, 2, 2], [0, 1, 2, 2, 2]]


def test_features_equal_brute_force():
    rng = np.random.default_rng(0)
    S = rng.standard_normal((3, 11, 4))
    np.testing.assert_array_equal(A.frame_features(S, 9, 5), loop_features(S, 9, 5))


def test_latent_groups_partition_the_frames():
    g = A.latent_groups(33, 8)
    assert [len(x) for x in g] == [1, 8, 8, 8, 8]
    assert sum(g, []) == list(range(33))
    assert A.latent_groups(9, 8) == [[0], list(range(1, 9))]
    with pytest.raises(ValueError):
        A.latent_groups(10, 8)


def test_mean_then_project_equals_project_then_mean():
    rng = np.random.default_rng(1)
    feat = rng.standard_normal((17, 24))
    lin = torch.nn.Linear(24, 6).double()
    by_frame = lin(torch.from_numpy(feat)).detach().numpy()
    want = np.stack([by_frame[g].mean(0) for g in A.latent_groups(17, 8)])
    got = lin(torch.from_numpy(A.latent_features(feat, 8))).detach().numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_pipeline_matches_torch_layers():
    acfg = synth.AUDIO_CONFIGS["toy"].replace(layers=2, state_frames=12, channels=8, hidden=16, tokens=4, dim=16)
    W = synth.weights_f32(synth.make_audio_weights(acfg))
    S = synth.audio_states(acfg, 2).astype(np.float64)
    got = A.audio_project(S, W, acfg)

    def lin(name):
        w = torch.from_numpy(W[name + ".w"].astype(np.float64))
        m = torch.nn.Linear(w.shape[1], w.shape[0]).double()
        with torch.no_grad():
            m.weight.copy_(w)
            m.bias.copy_(torch.from_numpy(W[name + ".b"].astype(np.float64)))
        return m

    norm = torch.nn.LayerNorm(acfg.dim, eps=acfg.eps).double()
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(W["projNorm.g"].astype(np.float64)))
        norm.bias.copy_(torch.from_numpy(W["projNorm.b"].astype(np.float64)))
    act = torch.nn.SiLU()
    for b in range(2):
        feat = loop_features(S[b], acfg.video_frames, acfg.window)
        rows = [torch.from_numpy(feat[0])] + [torch.from_numpy(feat[1 + 8 * i: 9 + 8 * i].mean(0))
                                             for i in range(acfg.latent_frames - 1)]
        h = [act(lin("proj1")(rows[0]))] + [act(lin("proj1vf")(r)) for r in rows[1:]]
        h = act(lin("proj2")(torch.stack(h)))
        y = lin("proj3")(h).reshape(acfg.latent_frames * acfg.tokens, acfg.dim)
        np.testing.assert_allclose(got[b], norm(y).detach().numpy(), rtol=0, atol=1e-10)


def test_token_order_and_norm_moments():
    acfg = synth.AUDIO_CONFIGS["toy"]
    W = synth.weights_f32(synth.make_audio_weights(acfg))
    W["proj3.w"] = np.zeros_like(W["proj3.w"])          # every latent frame gives the bias's tokens
    W["proj3.b"] = np.arange(acfg.tokens * acfg.dim, dtype=np.float32) % 97 * np.float32(0.1)
    W["projNorm.g"] = np.ones(acfg.dim, np.float32)
    W["projNorm.b"] = np.zeros(acfg.dim, np.float32)
    y = A.audio_project(synth.audio_states(acfg, 1), W, acfg)[0]
    assert y.shape == (acfg.latent_frames * acfg.tokens, acfg.dim)
    tok = W["proj3.b"].astype(np.float64).reshape(acfg.tokens, acfg.dim)
    want = (tok - tok.mean(1, keepdims=True)) / np.sqrt(tok.var(1, keepdims=True) + acfg.eps)
    for i in range(acfg.latent_frames):
        np.testing.assert_allclose(y[i * acfg.tokens:(i + 1) * acfg.tokens], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y.mean(1), 0, atol=1e-12)
