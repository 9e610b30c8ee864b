"""Float64 oracle of the re-noising sampler update and its counter-based noise.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: the audio-cpp page "SoulX-FlashHead", section "Variant
boundaries", says the distilled checkpoints (Lite among them) step with a
re-noising update rather than plain Euler, and does not write it out.

READING (the plainest flow-matching form, with the velocity convention
x_s = (1 - s) x0 + s eps, v = eps - x0 used by the Euler sampler):
    x0_hat = x - s v
    x'     = (1 - s') x0_hat + s' eps_new
with eps_new fresh standard-normal noise per step. With eps_new replaced by
the model's own noise estimate x + (1 - s) v this is the Euler update, and at
s' = 0 it is the Euler update whatever the noise (both pinned in tests).

The noise is counter-based so that any element of any step can be drawn
independently and reproducibly: the Philox-4x32 generator of Salmon, Moraes,
Dror and Shaw ("Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with
10 rounds, then the Box-Muller transform. Counter and key layout (READING;
the pages name no generator):
    element i (flat index over [C, F, H, W] of batch lane b) at step k:
    counter = (i // 4, b, k, 0), key = (seed mod 2^32, seed // 2^32);
    of the four output words w0..w3, element i takes pair p = (i mod 4) // 2,
    u_a = ((w_{2p} >> 8) + 1) / 2^24, u_b = ((w_{2p+1} >> 8) + 1) / 2^24 (in (0, 1]),
    r = sqrt(-2 ln u_a), theta = 2 pi u_b,
    eps = r cos(theta) for even i, r sin(theta) for odd i.
These 24-bit uniforms are exact in float32, so both sides start the
transform from the same values.

Pinned (tests/test_oracle_renoise.py): the generator's bijectivity on a counter
sample, key and counter sensitivity and avalanche, bit and byte uniformity;
the normal samples' moments and a Kolmogorov-Smirnov test; the update's two
Euler identities, zero-step identity and motion pinning.
"""
from __future__ import annotations

import numpy as np

from .dit import dit_flow, pin_motion, to64

__all__ = ["philox4x32", "noise_uniforms", "slice_noise", "renoise_step", "denoise_slice_renoise"]

# the generator's published constants: round multipliers and Weyl key increments
_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32(ctr, key, rounds=10):
    """Philox-4x32 of counters ctr [..., 4] under keys key [..., 2] (uint32
    values in any integer array), -> [..., 4] uint32.

    One round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 (64-bit products);
    c' = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key then advances by
    (W0, W1) mod 2^32 before the next round.
    """
    c = np.asarray(ctr, dtype=np.uint64) & _MASK
    k = np.asarray(key, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = (c[..., j].copy() for j in range(4))
    k0, k1 = np.broadcast_to(k[..., 0], c0.shape).copy(), np.broadcast_to(k[..., 1], c0.shape).copy()
    for r in range(rounds):
        p0 = np.uint64(_M0) * c0          # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if r + 1 < rounds:
            k0 = (k0 + np.uint64(_W0)) & np.uint64(_MASK)
            k1 = (k1 + np.uint64(_W1)) & np.uint64(_MASK)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def noise_uniforms(words):
    """24-bit uniforms in (0, 1] from 32-bit words: ((w >> 8) + 1) / 2^24."""
    return ((np.asarray(words, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) + 1.0) / 16777216.0


def slice_noise(seed, step, shape):
    """Standard-normal noise eps [B, C, F, H, W] of one step (layout above)."""
    B = shape[0]
    n = int(np.prod(shape[1:]))
    i = np.arange(n, dtype=np.uint64)
    out = np.empty((B, n))
    key = np.array([seed & _MASK, (seed >> 32) & _MASK], dtype=np.uint64)
    for b in range(B):
        g = i >> np.uint64(2)
        ctr = np.stack([g, np.full(n, b, np.uint64), np.full(n, step, np.uint64), np.zeros(n, np.uint64)], -1)
        w = philox4x32(ctr, key).astype(np.uint64)
        pair = ((i & np.uint64(3)) >> np.uint64(1)).astype(np.int64)
        ua = noise_uniforms(np.take_along_axis(w, (2 * pair)[:, None], 1)[:, 0])
        ub = noise_uniforms(np.take_along_axis(w, (2 * pair + 1)[:, None], 1)[:, 0])
        r = np.sqrt(-2.0 * np.log(ua))
        th = 2.0 * np.pi * ub
        out[b] = np.where((i & np.uint64(1)) == 0, r * np.cos(th), r * np.sin(th))
    return out.reshape(shape)


def renoise_step(latent, v, sigma, sigma_next, eps):
    """x' = (1 - s') (x - s v) + s' eps (READING above)."""
    s, s2 = float(sigma), float(sigma_next)
    x0 = to64(latent) - s * to64(v)
    return (1.0 - s2) * x0 + s2 * to64(eps)


def denoise_slice_renoise(noise, motion, audio, sigmas, W, cfg, seed):
    """As denoise_slice with the re-noising update; eps of step k from slice_noise(seed, k, ...)."""
    x = pin_motion(noise, motion)
    for k in range(len(sigmas) - 1):
        v = dit_flow(x, sigmas[k], audio, W, cfg)
        eps = slice_noise(seed, k, x.shape)
        x = pin_motion(renoise_step(x, v, sigmas[k], sigmas[k + 1], eps), motion)
    return x
