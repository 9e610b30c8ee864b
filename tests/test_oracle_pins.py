"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a library routine on a special
case, a closed form, an invariant, or brute force on tiny inputs, chosen so
that a dropped term, a wrong sign or index, or a transposed operand fails.
No GPU is needed.
"""
import cmath
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth

T64 = torch.float64


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float64)))


def tiny_cfg(**kw):
    base = dict(n_blocks=2, dim=24, n_heads=2, head_dim=12, ffn_dim=40, in_ch=4, out_ch=4,
                frames=3, height=2, width=3, motion_frames=1, audio_per_frame=4, freq_dim=16)
    base.update(kw)
    return synth.DiTConfig(**base)


def tiny_weights(cfg, seed=7, scale=1.0):
    W = synth.weights_f32(synth.make_weights(cfg, seed=seed))
    return {k: np.asarray(v, np.float64) * (scale if v.ndim == 2 and not k.endswith("mod") else 1.0)
            for k, v in W.items()}


rng = np.random.default_rng(2024)


# ---------------------------------------------------------------- elementary
def test_layer_norm_matches_torch():
    x = rng.standard_normal((3, 5, 37)) * 3 + 1.5
    g, b = rng.standard_normal(37), rng.standard_normal(37)
    ref = F.layer_norm(t64(x), (37,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(x, 1e-6), ref, rtol=0, atol=1e-12)
    ref = F.layer_norm(t64(x), (37,), t64(g), t64(b), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(x, 1e-6, g, b), ref, rtol=0, atol=1e-12)
    y = O.layer_norm(x, 0.0)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(-1), 1, atol=1e-12)


def test_rms_norm_matches_torch():
    x = rng.standard_normal((4, 6, 40)) * 2
    g = rng.standard_normal(40)
    ref = F.rms_norm(t64(x), (40,), t64(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=0, atol=1e-12)
    y = O.rms_norm(x, np.ones(40), 0.0)
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(-1)), 1, atol=1e-12)


def test_gelu_tanh_and_silu_match_torch():
    z = np.linspace(-9, 9, 1001)
    np.testing.assert_allclose(O.gelu_tanh(z), F.gelu(t64(z), approximate="tanh").numpy(),
                               rtol=0, atol=1e-14)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.gelu_tanh(z) - O.gelu_tanh(-z), z, atol=1e-12)
    np.testing.assert_allclose(O.silu(z), F.silu(t64(z)).numpy(), rtol=0, atol=1e-14)


def test_softmax_rows():
    s = rng.standard_normal((5, 9)) * 30
    p = O.softmax(s)
    np.testing.assert_allclose(p.sum(-1), 1, atol=1e-14)
    np.testing.assert_allclose(p, torch.softmax(t64(s), -1).numpy(), atol=1e-15)


def test_linear_matches_torch():
    x, w, b = rng.standard_normal((7, 11)), rng.standard_normal((5, 11)), rng.standard_normal(5)
    np.testing.assert_allclose(O.linear(x, w, b), F.linear(t64(x), t64(w), t64(b)).numpy(),
                               atol=1e-13)


# ---------------------------------------------------------------- time embedding
def test_sinusoid_closed_forms():
    e = O.sinusoid(np.array([0.0]), 16)
    np.testing.assert_array_equal(e[0, :8], 1.0)
    np.testing.assert_array_equal(e[0, 8:], 0.0)
    t = 731.25
    e = O.sinusoid(np.array([t]), 256)[0]
    for k in (0, 1, 57, 127):
        z = cmath.exp(1j * t * 10000.0 ** (-k / 128))
        assert abs(e[k] - z.real) < 1e-12 and abs(e[128 + k] - z.imag) < 1e-12


def test_time_embedding_matches_torch_layers():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    sig = np.array([1.0, 0.25])
    e, e0 = O.time_embedding(sig, W, cfg)
    emb = t64(O.sinusoid(1000.0 * sig, cfg.freq_dim))
    lin = lambda n: (lambda x: F.linear(x, t64(W[n + ".w"]), t64(W[n + ".b"])))
    e_ref = lin("time_out")(F.silu(lin("time_in")(emb)))
    e0_ref = lin("time_proj")(F.silu(e_ref)).reshape(2, 6, cfg.dim)
    np.testing.assert_allclose(e, e_ref.numpy(), atol=1e-13)
    np.testing.assert_allclose(e0, e0_ref.numpy(), atol=1e-13)


# ---------------------------------------------------------------- rotary
def test_rope_pair_split_and_angles():
    assert O.rope_pair_split(128) == (22, 21, 21)
    cfg = synth.CONFIGS["slice"]
    ang = O.rope_angles(cfg)
    assert ang.shape == (1280, 64)
    pos = O.token_positions(cfg)
    # pair 0 of each axis turns by exactly the token's position on that axis
    np.testing.assert_array_equal(ang[:, 0], pos[:, 0])
    np.testing.assert_array_equal(ang[:, 22], pos[:, 1])
    np.testing.assert_array_equal(ang[:, 43], pos[:, 2])
    # last frame pair: frequency 10^4^(-21/22); last column pair: 10^4^(-20/21)
    n = 2 * 256 + 3 * 16 + 7            # token at frame 2, row 3, column 7
    assert tuple(pos[n]) == (2, 3, 7)
    assert abs(ang[n, 21] - 2 * 10000.0 ** (-21 / 22)) < 1e-15
    assert abs(ang[n, 63] - 7 * 10000.0 ** (-20 / 21)) < 1e-15
    assert abs(ang[n, 30] - 3 * 10000.0 ** (-8 / 21)) < 1e-15


def test_rope_is_complex_multiplication():
    cfg = tiny_cfg()
    ang = O.rope_angles(cfg)
    x = rng.standard_normal((1, cfg.tokens, 2, cfg.head_dim))
    y = O.apply_rope(x, ang)
    for n in (0, 5, cfg.tokens - 1):
        for h in range(2):
            for j in range(cfg.head_dim // 2):
                z = complex(x[0, n, h, 2 * j], x[0, n, h, 2 * j + 1]) * cmath.exp(1j * ang[n, j])
                assert abs(y[0, n, h, 2 * j] - z.real) < 1e-12
                assert abs(y[0, n, h, 2 * j + 1] - z.imag) < 1e-12


def test_rope_invariants():
    cfg = tiny_cfg(frames=4, height=3, width=5)
    ang = O.rope_angles(cfg)
    x = rng.standard_normal((1, cfg.tokens, 1, cfg.head_dim))
    y = O.apply_rope(x, ang)
    # norm of every pair preserved
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]),
                               np.hypot(x[..., 0::2], x[..., 1::2]), atol=1e-12)
    # position (0,0,0) is the identity
    np.testing.assert_allclose(y[0, 0], x[0, 0], atol=0)
    # relative invariance: <R(p) q, R(p') k> depends on p - p' only
    q, k = rng.standard_normal(cfg.head_dim), rng.standard_normal(cfg.head_dim)
    pos = O.token_positions(cfg)
    idx = {tuple(p): i for i, p in enumerate(pos)}

    def dot(pq, pk):
        a = O.apply_rope(q[None, None, None], ang[idx[pq]][None])[0, 0, 0]
        b = O.apply_rope(k[None, None, None], ang[idx[pk]][None])[0, 0, 0]
        return a @ b
    assert abs(dot((2, 1, 3), (1, 0, 1)) - dot((1, 2, 4), (0, 1, 2))) < 1e-11
    assert abs(dot((3, 2, 4), (0, 0, 0)) - dot((3, 2, 4), (0, 0, 0))) == 0
    assert abs(dot((3, 1, 0), (2, 1, 0)) - dot((1, 0, 0), (0, 0, 0))) < 1e-11
    # moving along one axis turns only that axis's pairs
    nf, nr, nc = O.rope_pair_split(cfg.head_dim)
    d = ang[idx[(1, 2, 3)]] - ang[idx[(0, 2, 3)]]
    assert np.all(d[:nf] != 0) and np.all(d[nf:] == 0)
    d = ang[idx[(1, 2, 3)]] - ang[idx[(1, 1, 3)]]
    assert np.all(d[:nf] == 0) and np.all(d[nf:nf + nr] != 0) and np.all(d[nf + nr:] == 0)
    d = ang[idx[(1, 2, 3)]] - ang[idx[(1, 2, 2)]]
    assert np.all(d[:nf + nr] == 0) and np.all(d[nf + nr:] != 0)


# ---------------------------------------------------------------- attention
def test_attention_brute_force_loops():
    q = rng.standard_normal((1, 2, 5, 4))
    k = rng.standard_normal((1, 2, 7, 4))
    v = rng.standard_normal((1, 2, 7, 3))
    o = O.attention(q, k, v)
    for h in range(2):
        for i in range(5):
            s = [sum(q[0, h, i, d] * k[0, h, j, d] for d in range(4)) / 2.0 for j in range(7)]
            w = [math.exp(x) for x in s]
            tot = sum(w)
            for d in range(3):
                ref = sum(w[j] * v[0, h, j, d] for j in range(7)) / tot
                assert abs(o[0, h, i, d] - ref) < 1e-12


def test_attention_matches_sdpa_and_invariants():
    q = rng.standard_normal((2, 3, 16, 8)) * 2
    k = rng.standard_normal((2, 3, 16, 8)) * 2
    v = rng.standard_normal((2, 3, 16, 8))
    ref = F.scaled_dot_product_attention(t64(q), t64(k), t64(v)).numpy()
    o = O.attention(q, k, v)
    np.testing.assert_allclose(o, ref, atol=1e-12)
    # q = 0: uniform weights, the mean of v
    np.testing.assert_allclose(O.attention(np.zeros_like(q), k, v),
                               np.broadcast_to(v.mean(2, keepdims=True), v.shape), atol=1e-13)
    # permuting keys and values together changes nothing; permuting queries permutes rows
    p = rng.permutation(16)
    np.testing.assert_allclose(O.attention(q, k[:, :, p], v[:, :, p]), o, atol=1e-13)
    np.testing.assert_allclose(O.attention(q[:, :, p], k, v), o[:, :, p], atol=1e-13)


def test_cross_attention_modes():
    cfg = tiny_cfg(frames=3)
    W = tiny_weights(cfg)
    Wb = O.block_weights(W, 0)
    B = 2
    h3 = rng.standard_normal((B, cfg.tokens, cfg.dim))
    a = rng.standard_normal((B, cfg.audio_tokens, cfg.dim))
    kc, vc = O.audio_kv(a, Wb, cfg)
    loc = O.cross_attention(h3, kc, vc, Wb, cfg)
    full = O.cross_attention(h3, kc, vc, Wb, cfg.replace(cross_full=True))
    assert np.abs(loc - full).max() > 1e-3
    # frame-local = full attention under a block mask (library routine)
    qc = O.rms_norm(O.linear(h3, Wb["cq.w"], Wb["cq.b"]), Wb["norm_cq.g"], cfg.eps)
    hw = cfg.height * cfg.width
    fq = np.arange(cfg.tokens) // hw
    fk = np.arange(cfg.audio_tokens) // cfg.audio_per_frame
    mask = torch.from_numpy(fq[:, None] == fk[None, :])
    sp = lambda x: t64(O.split_heads(x, cfg.n_heads))
    ref = F.scaled_dot_product_attention(sp(qc), sp(kc), sp(vc), attn_mask=mask)
    np.testing.assert_allclose(loc, O.merge_heads(ref.numpy()), atol=1e-12)
    # one latent frame: both modes coincide
    c1 = cfg.replace(frames=1)
    k1, v1 = kc[:, :4], vc[:, :4]
    np.testing.assert_allclose(O.cross_attention(h3[:, :hw], k1, v1, Wb, c1),
                               O.cross_attention(h3[:, :hw], k1, v1, Wb, c1.replace(cross_full=True)),
                               atol=1e-13)
    # the same audio block in every frame: duplicate keys cancel, modes coincide
    rep = np.tile(a[:, :cfg.audio_per_frame], (1, cfg.frames, 1))
    kr, vr = O.audio_kv(rep, Wb, cfg)
    np.testing.assert_allclose(O.cross_attention(h3, kr, vr, Wb, cfg),
                               O.cross_attention(h3, kr, vr, Wb, cfg.replace(cross_full=True)),
                               atol=1e-12)


# ---------------------------------------------------------------- block
def _branch_off(Wb, *names):
    Wb = dict(Wb)
    for n in names:
        Wb[n] = np.zeros_like(Wb[n])
    return Wb


def test_block_identity_pins():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    Wb = O.block_weights(W, 0)
    ang = O.rope_angles(cfg)
    x = rng.standard_normal((2, cfg.tokens, cfg.dim))
    a = rng.standard_normal((2, cfg.audio_tokens, cfg.dim))
    e0 = rng.standard_normal((2, 6, cfg.dim))
    Z = _branch_off(Wb, "o.w", "o.b", "co.w", "co.b", "ffn2.w", "ffn2.b")
    np.testing.assert_array_equal(O.dit_block(x, e0, a, Z, cfg, ang), x)
    e0z = e0.copy()
    e0z[:, 2] = -Wb["mod"][2]
    e0z[:, 5] = -Wb["mod"][5]
    Z = _branch_off(Wb, "co.w", "co.b")
    np.testing.assert_allclose(O.dit_block(x, e0z, a, Z, cfg, ang), x, atol=1e-15)
    assert np.abs(O.dit_block(x, e0, a, Wb, cfg, ang) - x).max() > 1e-2


def test_block_branches_match_torch_layers():
    """Each residual branch alone, rebuilt from torch library layers."""
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    Wb = O.block_weights(W, 1)
    ang = O.rope_angles(cfg)
    B, N, D, nh, dh = 2, cfg.tokens, cfg.dim, cfg.n_heads, cfg.head_dim
    x = rng.standard_normal((B, N, D))
    a = rng.standard_normal((B, cfg.audio_tokens, D))
    e0 = rng.standard_normal((B, 6, D)) * 0.3
    m = t64(Wb["mod"])[None] + t64(e0)
    X = t64(x)
    lin = lambda n, h: F.linear(h, t64(Wb[n + ".w"]), t64(Wb[n + ".b"]))
    ln = lambda h: F.layer_norm(h, (D,), eps=cfg.eps)
    # FFN branch
    h = ln(X) * (1 + m[:, 4:5]) + m[:, 3:4]
    ffn = lin("ffn2", F.gelu(lin("ffn1", h), approximate="tanh"))
    got = O.dit_block(x, e0, a, _branch_off(Wb, "o.w", "o.b", "co.w", "co.b"), cfg, ang)
    np.testing.assert_allclose(got, (X + m[:, 5:6] * ffn).numpy(), atol=1e-12)
    # self-attention branch, rotary through torch complex numbers
    h = ln(X) * (1 + m[:, 1:2]) + m[:, 0:1]
    qkv = lin("qkv", h)
    q = F.rms_norm(qkv[..., :D], (D,), t64(Wb["norm_q.g"]), eps=cfg.eps)
    k = F.rms_norm(qkv[..., D:2 * D], (D,), t64(Wb["norm_k.g"]), eps=cfg.eps)
    v = qkv[..., 2 * D:]
    rot = torch.polar(torch.ones_like(t64(ang)), t64(ang))[None, :, None, :]

    def rope(t):
        c = torch.view_as_complex(t.reshape(B, N, nh, dh // 2, 2).contiguous()) * rot
        return torch.view_as_real(c).reshape(B, N, nh, dh).transpose(1, 2)
    o = F.scaled_dot_product_attention(rope(q), rope(k), v.reshape(B, N, nh, dh).transpose(1, 2))
    sa = lin("o", o.transpose(1, 2).reshape(B, N, D))
    got = O.dit_block(x, e0, a, _branch_off(Wb, "co.w", "co.b", "ffn2.w", "ffn2.b"), cfg, ang)
    np.testing.assert_allclose(got, (X + m[:, 2:3] * sa).numpy(), atol=1e-12)
    # cross-attention branch (ungated), through a masked SDPA
    h3 = F.layer_norm(X, (D,), t64(Wb["norm3.g"]), t64(Wb["norm3.b"]), eps=cfg.eps)
    qc = F.rms_norm(lin("cq", h3), (D,), t64(Wb["norm_cq.g"]), eps=cfg.eps)
    kv = lin("ckv", t64(a))
    kc = F.rms_norm(kv[..., :D], (D,), t64(Wb["norm_ck.g"]), eps=cfg.eps)
    vc = kv[..., D:]
    fq = torch.arange(N) // (cfg.height * cfg.width)
    fk = torch.arange(cfg.audio_tokens) // cfg.audio_per_frame
    sp = lambda t: t.reshape(B, -1, nh, dh).transpose(1, 2)
    oc = F.scaled_dot_product_attention(sp(qc), sp(kc), sp(vc), attn_mask=fq[:, None] == fk[None])
    ca = lin("co", oc.transpose(1, 2).reshape(B, N, D))
    got = O.dit_block(x, e0, a, _branch_off(Wb, "o.w", "o.b", "ffn2.w", "ffn2.b"), cfg, ang)
    np.testing.assert_allclose(got, (X + ca).numpy(), atol=1e-12)


# ---------------------------------------------------------------- layout, sampler
def test_patchify_order_and_round_trip():
    cfg = tiny_cfg()
    lat = rng.standard_normal((2, cfg.in_ch, cfg.frames, cfg.height, cfg.width))
    tok = O.patchify(lat)
    pos = O.token_positions(cfg)
    for n in (0, 4, cfg.tokens - 1):
        f, r, c = pos[n]
        np.testing.assert_array_equal(tok[:, n], lat[:, :, f, r, c])
    np.testing.assert_array_equal(O.unpatchify(tok, cfg), lat)


def _sampler_case(scale=1.0):
    cfg = tiny_cfg(frames=3, motion_frames=1)
    W = tiny_weights(cfg)
    B = 2
    noise = rng.standard_normal((B, cfg.in_ch, cfg.frames, cfg.height, cfg.width))
    mot = rng.standard_normal((B, cfg.in_ch, cfg.motion_frames, cfg.height, cfg.width))
    a = rng.standard_normal((B, cfg.audio_tokens, cfg.dim))
    return cfg, W, noise, mot, a


def test_sampler_zero_steps_and_zero_step_size():
    cfg, W, noise, mot, a = _sampler_case()
    out = O.denoise_slice(noise, mot, a, [0.7], W, cfg)
    np.testing.assert_array_equal(out, O.pin_motion(noise, mot))
    out = O.denoise_slice(noise, mot, a, [0.5, 0.5, 0.5], W, cfg)
    np.testing.assert_array_equal(out, O.pin_motion(noise, mot))


def test_sampler_constant_velocity_closed_form():
    cfg, W, noise, mot, a = _sampler_case()
    W = dict(W)
    W["head.w"] = np.zeros_like(W["head.w"])
    sig = [1.0, 0.75, 0.5, 0.25, 0.0]
    out = O.denoise_slice(noise, mot, a, sig, W, cfg)
    exp = noise + (sig[-1] - sig[0]) * W["head.b"][None, :, None, None, None]
    np.testing.assert_allclose(out[:, :, 1:], exp[:, :, 1:], atol=1e-14)
    np.testing.assert_array_equal(out[:, :, :1], mot)


def test_sampler_motion_pinned_and_lanes_independent():
    cfg, W, noise, mot, a = _sampler_case()
    sig = [1.0, 0.5, 0.0]
    out = O.denoise_slice(noise, mot, a, sig, W, cfg)
    np.testing.assert_array_equal(out[:, :, :cfg.motion_frames], mot)
    one = O.denoise_slice(noise[1:], mot[1:], a[1:], sig, W, cfg)
    np.testing.assert_allclose(out[1:], one, atol=1e-13)
    # it moved: the flow is not zero
    assert np.abs(out - O.pin_motion(noise, mot)).max() > 1e-2
    # the first step from the pinned noise is one flow evaluation
    v = O.dit_flow(O.pin_motion(noise, mot), 1.0, a, W, cfg)
    x1 = O.pin_motion(O.pin_motion(noise, mot) - 0.5 * v, mot)
    v1 = O.dit_flow(x1, 0.5, a, W, cfg)
    np.testing.assert_allclose(out, O.pin_motion(x1 - 0.5 * v1, mot), atol=1e-13)


def test_renoise_with_own_estimate_equals_euler():
    """x0 = x - s v, eps = x + (1 - s) v; (1 - s') x0 + s' eps = x + (s' - s) v."""
    x = rng.standard_normal(50)
    v = rng.standard_normal(50)
    for s, s2 in ((1.0, 0.75), (0.75, 0.5), (0.25, 0.0)):
        x0, eps = x - s * v, x + (1 - s) * v
        np.testing.assert_allclose((1 - s2) * x0 + s2 * eps, O.euler_step(x, v, s, s2), atol=1e-14)


def test_flow_head_is_modulated_output_norm():
    """With every block's output weights zeroed the DiT is patch -> head:
    v = (LN(x)(1+scale)+shift) W_h^T + b_h with (shift, scale) = head.mod + e."""
    cfg, W, noise, mot, a = _sampler_case()
    W = dict(W)
    for i in range(cfg.n_blocks):
        for n in ("o.w", "o.b", "co.w", "co.b", "ffn2.w", "ffn2.b"):
            W[f"blocks.{i}.{n}"] = np.zeros_like(W[f"blocks.{i}.{n}"])
    lat = O.pin_motion(noise, mot)
    v = O.dit_flow(lat, 0.6, a, W, cfg)
    e, _ = O.time_embedding(np.full(2, 0.6), W, cfg)
    tok = torch.from_numpy(np.moveaxis(lat, 1, -1).reshape(2, -1, cfg.in_ch))
    x = F.linear(tok, t64(W["patch.w"]), t64(W["patch.b"]))
    hm = t64(W["head.mod"])[None] + t64(e)[:, None]
    h = F.layer_norm(x, (cfg.dim,), eps=cfg.eps) * (1 + hm[:, 1:2]) + hm[:, 0:1]
    ref = F.linear(h, t64(W["head.w"]), t64(W["head.b"])).numpy()
    ref = np.moveaxis(ref.reshape(2, cfg.frames, cfg.height, cfg.width, -1), -1, 1)
    np.testing.assert_allclose(v, ref, atol=1e-12)


def test_parameter_count_is_1_3b():
    """The toolkit page and the press release call FlashHead a 1.3B model."""
    cfg = synth.CONFIGS["slice"]
    n = sum(int(np.prod(s)) for _, s, _ in synth.param_specs(cfg))
    blocks = sum(int(np.prod(s)) for name, s, _ in synth.param_specs(cfg) if name.startswith("blocks."))
    assert 1.30e9 <= blocks <= 1.45e9 and 1.30e9 <= n <= 1.45e9


def test_rel_err_excludes_motion_frames():
    r = np.ones((1, 2, 3, 2, 2))
    g = r.copy()
    g[:, :, 0] += 5.0
    assert O.rel_err(g, r, motion_frames=1) == 0.0
    assert O.rel_err(g, r) == 5.0


def test_float32_working_dtype_follows_the_float64_path():
    """working_dtype(np.float32) (the fp32 CPU baseline) runs every statement in
    float32 -- no silent promotion back to float64 -- and agrees with the
    float64 path to float32 rounding on a small slice and on one block of the
    real width. The default outside the scope stays float64."""
    cfg, W, noise, mot, a = _sampler_case()
    sig = [1.0, 0.5, 0.0]
    ref = O.denoise_slice(noise, mot, a, sig, W, cfg)
    with O.working_dtype(np.float32):
        got = O.denoise_slice(noise, mot, a, sig, W, cfg)
        v = O.dit_flow(O.pin_motion(noise, mot), 1.0, a, W, cfg)
    assert got.dtype == np.float32 and v.dtype == np.float32
    assert O.rel_err(got, ref, cfg.motion_frames) < 1e-5
    assert O.denoise_slice(noise, mot, a, sig, W, cfg).dtype == np.float64
    # one block at width 256 with 2 heads of 128 (the toy DiT's block)
    tc = synth.CONFIGS["toy"]
    Wt = synth.weights_f32(synth.make_weights(tc, blocks=[0]))
    x = rng.standard_normal((1, tc.tokens, tc.dim))
    e = rng.standard_normal((1, tc.dim))
    aud = rng.standard_normal((1, tc.audio_tokens, tc.dim))
    want = O.dit_block_from_temb(x, e, aud, Wt, 0, tc)
    with O.working_dtype(np.float32):
        have = O.dit_block_from_temb(x, e, aud, Wt, 0, tc)
    assert have.dtype == np.float32
    assert O.rel_err(have - x, want - x) < 1e-5


def test_err_stats_closed_forms():
    """The three error figures on a constructed case: ref = 1 everywhere on
    non-motion frames, got = ref except one element off by 0.5 and a 1e-3
    offset on 1 % of the elements."""
    ref = np.ones((1, 2, 3, 10, 10))
    got = ref.copy()
    got[:, :, 0] = 7.0                          # motion frame: ignored
    flat = got[:, :, 1:].reshape(-1)
    n = flat.size                                # 400
    flat_idx = np.arange(n)
    view = got[:, :, 1:].reshape(-1)
    view[flat_idx[:4]] += 1e-3                   # 1 %
    view[n - 1] += 0.5
    got[:, :, 1:] = view.reshape(got[:, :, 1:].shape)
    s = O.err_stats(got, ref, 1)
    assert s["max"] == pytest.approx(0.5)
    assert s["rel_l2"] == pytest.approx(np.sqrt(4e-6 + 0.25) / np.sqrt(n))
    assert 1e-3 - 1e-12 <= s["p999"] <= 0.5      # the 99.9th percentile sits between the offsets and the outlier
    assert O.err_stats(got, ref, 1)["max"] == O.rel_err(got, ref, 1)
