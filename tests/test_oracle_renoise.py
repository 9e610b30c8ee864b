"""Pins of the re-noising sampler oracle (oracle/renoise.py): the counter-based
generator, the normal transform and the update, against properties the
definitions fix (no GPU).

The generator is checked by what any correct Philox-4x32-10 must satisfy: a
bijection of the counter for a fixed key, full dependence on every key and
counter bit (half the output bits flip, on average, for one flipped input bit),
uniform bits and bytes; dropping a key or counter term, a wrong word order or
too few rounds fails the avalanche or the bijection test.
"""
import numpy as np
import pytest
from scipy import stats

import oracle as O
from oracle import renoise as R
import synth


def _ctr(n, base=0):
    g = np.arange(base, base + n, dtype=np.uint64)
    return np.stack([g & 0xFFFFFFFF, g >> 32, np.full(n, 3, np.uint64), np.full(n, 11, np.uint64)], -1)


KEY = np.array([0x1234ABCD, 0x0F0F1E1E], dtype=np.uint64)


def _pack(w):
    w = w.astype(np.uint64)
    return (w[:, 0] << np.uint64(96 - 64)) ^ w[:, 1], (w[:, 2] << np.uint64(32)) | w[:, 3]


def test_philox_is_a_bijection_on_a_counter_sample():
    out = R.philox4x32(_ctr(1 << 16), KEY)
    rows = {tuple(r) for r in out.tolist()}
    assert len(rows) == 1 << 16
    # and distinct keys give distinct streams
    out2 = R.philox4x32(_ctr(1 << 12), KEY ^ np.array([1, 0], dtype=np.uint64))
    assert not np.any(np.all(out2 == out[: 1 << 12], axis=1))


def _bits(x):
    return np.unpackbits(x.astype(">u4").view(np.uint8).reshape(x.shape[0], -1), axis=1)


@pytest.mark.parametrize("word", range(6))  # counter words 0..3, key words 0..1
def test_philox_avalanche_on_every_input_word(word):
    n = 2048
    ctr = _ctr(n, base=77) ^ np.uint64(0)
    ctr = (np.random.default_rng(word).integers(0, 2**32, (n, 4), dtype=np.uint64))
    key = np.random.default_rng(100 + word).integers(0, 2**32, (n, 2), dtype=np.uint64)
    base = _bits(R.philox4x32(ctr, key))
    flips = []
    for bit in range(0, 32, 3):
        c2, k2 = ctr.copy(), key.copy()
        if word < 4:
            c2[:, word] ^= np.uint64(1 << bit)
        else:
            k2[:, word - 4] ^= np.uint64(1 << bit)
        d = (base != _bits(R.philox4x32(c2, k2))).sum(1)
        flips.append(d.mean())
        assert 60.0 < d.mean() < 68.0, (word, bit, d.mean())
    assert 62.5 < np.mean(flips) < 65.5


def test_philox_round_count_matters():
    """Two rounds do not mix a low counter bit into every output word; ten do."""
    ctr = _ctr(4096)
    c2 = ctr.copy()
    c2[:, 2] ^= np.uint64(1)
    for rounds, mixes in ((2, False), (10, True)):
        d = R.philox4x32(ctr, KEY, rounds) != R.philox4x32(c2, KEY, rounds)
        assert bool(np.all(d.mean(0) > 0.99)) == mixes


def test_philox_bits_and_bytes_are_uniform():
    out = R.philox4x32(_ctr(1 << 16), KEY)
    bits = _bits(out)
    n = bits.shape[0]
    assert np.all(np.abs(bits.mean(0) - 0.5) < 5 * 0.5 / np.sqrt(n))
    counts = np.bincount(out.view(np.uint8).ravel(), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_uniforms_are_24_bit_and_never_zero():
    w = np.array([0, 255, 256, 0xFFFFFFFF], dtype=np.uint64)
    u = R.noise_uniforms(w)
    np.testing.assert_array_equal(u, [1 / 2**24, 1 / 2**24, 2 / 2**24, 1.0])
    u = R.noise_uniforms(np.random.default_rng(1).integers(0, 2**32, 10000, dtype=np.uint64))
    assert np.all(u.astype(np.float32) == u) and np.all(u > 0) and np.all(u <= 1)  # exact in float32


def test_slice_noise_is_standard_normal():
    eps = R.slice_noise(42, 0, (2, 16, 5, 16, 16)).ravel()
    assert abs(eps.mean()) < 5 / np.sqrt(eps.size)
    assert abs(eps.var() - 1) < 5 * np.sqrt(2 / eps.size)
    assert stats.kstest(eps, "norm").pvalue > 1e-3
    # the cos and sin halves of each Box-Muller pair are uncorrelated
    assert abs(np.corrcoef(eps[0::2], eps[1::2])[0, 1]) < 5 / np.sqrt(eps.size / 2)


def test_slice_noise_is_counter_addressed():
    a = R.slice_noise(7, 2, (3, 4, 2, 3, 4))
    np.testing.assert_array_equal(R.slice_noise(7, 2, (1, 4, 2, 3, 4))[0], a[0])  # lane 0 alone
    assert not np.allclose(a[0], a[1])                                               # lanes differ
    assert not np.allclose(R.slice_noise(7, 3, a.shape), a)                           # steps differ
    assert not np.allclose(R.slice_noise(8, 2, a.shape), a)                           # seeds differ
    assert not np.allclose(R.slice_noise(7 + (1 << 32), 2, a.shape), a)               # high seed word used
    # element i takes word pair (i mod 4) // 2 of counter i // 4: recompute one element by hand
    w = R.philox4x32(np.array([[5 // 4, 1, 2, 0]], np.uint64), np.array([7, 0], np.uint64))[0]
    ua, ub = R.noise_uniforms(w[0:2])  # element 5: pair (5 mod 4) // 2 = 0, odd -> sin
    ref = np.sqrt(-2 * np.log(ua)) * np.sin(2 * np.pi * ub)
    assert a[1].ravel()[5] == pytest.approx(ref, rel=1e-15)


def test_renoise_with_own_noise_estimate_is_euler():
    rng = np.random.default_rng(5)
    x, v = rng.standard_normal(64), rng.standard_normal(64)
    for s, s2 in ((1.0, 0.75), (0.75, 0.5), (0.5, 0.25)):
        got = R.renoise_step(x, v, s, s2, x + (1 - s) * v)
        np.testing.assert_allclose(got, O.euler_step(x, v, s, s2), atol=1e-13)


def test_renoise_last_step_is_euler_for_any_noise():
    rng = np.random.default_rng(6)
    x, v, eps = rng.standard_normal((3, 64))
    np.testing.assert_allclose(R.renoise_step(x, v, 0.25, 0.0, eps), O.euler_step(x, v, 0.25, 0.0), atol=1e-15)


def _case():
    cfg = synth.DiTConfig(n_blocks=1, dim=24, n_heads=2, head_dim=12, ffn_dim=40, in_ch=4, out_ch=4,
                          frames=3, height=2, width=3, motion_frames=1, audio_per_frame=4, freq_dim=16)
    W = {k: np.asarray(v, np.float64) for k, v in synth.weights_f32(synth.make_weights(cfg, seed=3)).items()}
    rng = np.random.default_rng(9)
    noise = rng.standard_normal((2, 4, 3, 2, 3))
    mot = rng.standard_normal((2, 4, 1, 2, 3))
    aud = rng.standard_normal((2, cfg.audio_tokens, cfg.dim))
    return cfg, W, noise, mot, aud


def test_renoise_slice_identities():
    cfg, W, noise, mot, aud = _case()
    # zero steps: the pinned input
    np.testing.assert_array_equal(R.denoise_slice_renoise(noise, mot, aud, [0.6], W, cfg, 1), O.pin_motion(noise, mot))
    # one step to sigma 0 is the Euler step
    np.testing.assert_allclose(R.denoise_slice_renoise(noise, mot, aud, [1.0, 0.0], W, cfg, 1),
                               O.denoise_slice(noise, mot, aud, [1.0, 0.0], W, cfg), atol=1e-13)
    # a four-step run keeps the motion frames bitwise and differs from Euler (fresh noise enters)
    sig = [1.0, 0.75, 0.5, 0.25, 0.0]
    out = R.denoise_slice_renoise(noise, mot, aud, sig, W, cfg, 1)
    np.testing.assert_array_equal(out[:, :, :1], mot)
    assert not np.allclose(out, O.denoise_slice(noise, mot, aud, sig, W, cfg))
    # step k's update uses exactly slice_noise(seed, k): rebuild the last step by hand
    x = R.denoise_slice_renoise(noise, mot, aud, sig[:4], W, cfg, 1)
    v = O.dit_flow(x, 0.25, aud, W, cfg)
    np.testing.assert_allclose(out, O.pin_motion(O.euler_step(x, v, 0.25, 0.0), mot), atol=1e-12)


def test_weyl_key_increments_are_their_closed_forms():
    """The key schedule adds floor(2^32 (phi - 1)) and floor(2^32 (sqrt 3 - 1))."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    phi_m1 = (Decimal(5).sqrt() - 1) / 2
    sqrt3_m1 = Decimal(3).sqrt() - 1
    assert R._W0 == int(phi_m1 * 2**32)
    assert R._W1 == int(sqrt3_m1 * 2**32)


def test_philox_is_ten_keyed_rounds():
    """R rounds = one round under key k, then k + W, ..., k + (R-1) W (mod 2^32)."""
    ctr = np.random.default_rng(3).integers(0, 2**32, (512, 4), dtype=np.uint64)
    key = np.random.default_rng(4).integers(0, 2**32, (512, 2), dtype=np.uint64)
    w = np.array([R._W0, R._W1], dtype=np.uint64)
    c = ctr
    for r in range(10):
        c = R.philox4x32(c, (key + np.uint64(r) * w) & np.uint64(0xFFFFFFFF), rounds=1).astype(np.uint64)
    np.testing.assert_array_equal(c, R.philox4x32(ctr, key))
    # and the one-round map is the published mixing step on a hand case
    one = R.philox4x32(np.array([[1, 2, 3, 4]], np.uint64), np.array([5, 6], np.uint64), rounds=1)[0]
    p0, p1 = 0xD2511F53 * 1, 0xCD9E8D57 * 3
    assert list(one) == [(p1 >> 32) ^ 2 ^ 5, p1 & 0xFFFFFFFF, (p0 >> 32) ^ 4 ^ 6, p0 & 0xFFFFFFFF]


def test_philox_matches_the_published_known_answer_vectors():
    """The generator equals Random123's published Philox-4x32-10 known-answer
    vectors (tests/golden/philox4x32_10_kat.txt): all-zero and all-ones
    counter/key, and the digits-of-pi case."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_10_kat.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(t, 16) for t in r]
        ctr, key, want = v[0:4], v[4:6], v[6:10]
        got = R.philox4x32(np.array([ctr], dtype=np.uint32), np.array(key, dtype=np.uint32))
        assert [int(x) for x in np.asarray(got).ravel()] == want
