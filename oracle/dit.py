"""Float64 numpy oracle of the FlashHead Lite DiT and its Euler sampler.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, smoke() and the
bench's cpu_baseline leg call this; the product path must not.

What the pages fix, and where:
  * gizai:flashhead reference page, overview paragraph: a Wan-style
    transformer of 30 blocks of width 1536 with 12 heads, rotary over frame,
    row and column, predicts the flow of a noisy latent of 5 frames of 16x16
    whose first latent frames are the previous slice's motion, in 4 steps;
    audio enters as 5 latent frames of 32 audio tokens.
  * same page, type FlashHead: ``patch`` and ``head`` are Linear layers;
    ``headMods`` holds, at each step, the output norm's shift and scale
    ([2, 1536] F32); ``cos``/``sin`` hold the rotary angles per token row,
    [1280, 768] F32, pair d of head h at column h*64 + d (so one angle per
    (token, pair), the same for every head).
  * SoulX-FlashHead audio-cpp page, section "Generate": 4 denoising steps;
    section "Variant boundaries": DiT intermediates are F32 in the native
    port, with small differences from the BF16 original expected.
  * Toolkit page "SoulX-FlashHead -- Talking Head Video Generation",
    comparison table: a diffusion model distilled to 4 steps.

The inside of a "Wan-style" block is not written out on any page. The plain
reading taken here (every READING below) is the pre-norm adaLN block: a
modulated LayerNorm before self-attention and before the FFN, each branch
gated by a modulation row; an affine LayerNorm before an ungated audio
cross-attention; q/k RMSNorm over the full width; 3-D rotary on adjacent
dimension pairs; tanh-GELU FFN; sinusoidal timestep embedding through a
two-layer SiLU MLP, projected to six modulation rows per block.

Arithmetic is float64 throughout by default; bf16 matrices arrive as exact
float values. ``working_dtype(np.float32)`` runs the same statements in
float32 (the plain fp32 CPU model timed as a baseline); tests pin it to the
float64 path on small inputs.
"""
from __future__ import annotations

import contextlib
import math

import numpy as np

__all__ = [
    "working_dtype", "linear", "silu", "sinusoid", "time_embedding", "layer_norm", "modulate",
    "rms_norm", "gelu_tanh", "token_positions", "rope_pair_split", "rope_angles",
    "apply_rope", "softmax", "attention", "split_heads", "merge_heads",
    "self_attention", "audio_kv", "cross_attention", "dit_block",
    "dit_block_from_temb", "patchify", "unpatchify", "dit_flow", "pin_motion",
    "euler_step", "denoise_slice", "block_weights", "to64", "rel_err", "err_stats",
]


_WORK = np.dtype(np.float64)


@contextlib.contextmanager
def working_dtype(dtype):
    """Run the oracle's arithmetic in `dtype` (float64 outside this scope)."""
    global _WORK
    old, _WORK = _WORK, np.dtype(dtype)
    try:
        yield
    finally:
        _WORK = old


def to64(a):
    """a as an array of the working dtype (float64 unless working_dtype says otherwise)."""
    return np.asarray(a, dtype=_WORK)


# ----------------------------------------------------------------------------
# elementary layers
# ----------------------------------------------------------------------------
def linear(x, w, b=None):
    """y = x W^T + b with W stored [out, in] (the pages' ``N.Linear``)."""
    y = to64(x) @ to64(w).T
    if b is not None:
        y = y + to64(b)
    return y


def silu(x):
    x = to64(x)
    return x / (1.0 + np.exp(-x))


def gelu_tanh(z):
    """READING (the FFN activation is not on the pages): tanh-approximated GELU,
    0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    z = to64(z)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def layer_norm(x, eps, g=None, b=None):
    """LayerNorm over the last axis with population variance.

    READING: eps = 1e-6; the modulated norms carry no affine (the FlashHead type
    on the gizai:flashhead page keeps ``ones``/``zeros`` tensors, read as the
    parameters of affine-free norms); the norm before cross-attention is affine.
    """
    x = to64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if g is not None:
        y = y * to64(g)
    if b is not None:
        y = y + to64(b)
    return y


def modulate(h, shift, scale):
    """adaLN: h (1 + scale) + shift, with shift/scale [B, D] broadcast over tokens."""
    return to64(h) * (1.0 + to64(scale)[:, None, :]) + to64(shift)[:, None, :]


def rms_norm(x, g, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    READING: applied to q and k over the full model width before the head
    split (Wan-style), eps = 1e-6.
    """
    x = to64(x)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * to64(g)


def softmax(s, axis=-1):
    s = to64(s)
    m = s.max(axis=axis, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=axis, keepdims=True)


# ----------------------------------------------------------------------------
# timestep embedding and modulation (gizai:flashhead page, FlashHead.headMods)
# ----------------------------------------------------------------------------
def sinusoid(t, dim):
    """[B] -> [B, dim]: [cos(t w_k) | sin(t w_k)], w_k = 10000^(-k/(dim/2)).

    READING (silent on the pages): the plain sinusoidal embedding, cosines first.
    """
    t = to64(t).reshape(-1)
    half = dim // 2
    w = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    ang = t[:, None] * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def time_embedding(sigma, W, cfg):
    """sigma [B] -> (e [B, D], e0 [B, 6, D]).

    READING: the timestep is t = 1000 sigma; e = Linear(SiLU(Linear(sin(t)))),
    e0 = Linear(SiLU(e)) split into six rows. Each step recomputes them, as
    the gizai:flashhead page keeps the output norm's shift/scale per step.
    """
    t = 1000.0 * to64(sigma).reshape(-1)
    emb = sinusoid(t, cfg.freq_dim)
    e = linear(silu(linear(emb, W["time_in.w"], W["time_in.b"])), W["time_out.w"], W["time_out.b"])
    e0 = linear(silu(e), W["time_proj.w"], W["time_proj.b"]).reshape(-1, 6, cfg.dim)
    return e, e0


# ----------------------------------------------------------------------------
# 3-D rotary (gizai:flashhead page, FlashHead.cos / FlashHead.sin)
# ----------------------------------------------------------------------------
def token_positions(cfg):
    """[N, 3] integer (frame, row, column) of each token, tokens in (f, r, c)
    row-major order; motion frames are frames 0..Fm-1 like any other."""
    f, r, c = np.meshgrid(np.arange(cfg.frames), np.arange(cfg.height), np.arange(cfg.width),
                          indexing="ij")
    return np.stack([f.ravel(), r.ravel(), c.ravel()], axis=1)


def rope_pair_split(head_dim):
    """Pairs per axis (frame, row, column). READING: rows and columns get
    head_dim//6 pairs each, the frame axis the rest (22/21/21 at 128)."""
    pairs = head_dim // 2
    pr = head_dim // 6
    return pairs - 2 * pr, pr, pr


def rope_angles(cfg):
    """[N, head_dim/2] angle of each (token, pair); the same for every head.

    Pair j of axis a (local index j_a, n_a pairs on that axis) turns by
    pos_a * theta^(-j_a / n_a), theta = 10^4 (READING: the usual rotary base).
    """
    pos = token_positions(cfg).astype(np.float64)
    cols = []
    for axis, n in enumerate(rope_pair_split(cfg.head_dim)):
        freq = cfg.rope_theta ** (-np.arange(n, dtype=np.float64) / n)
        cols.append(pos[:, axis:axis + 1] * freq[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(x, ang):
    """x [B, N, nh, dh]; pair j is dims (2j, 2j+1) (READING: adjacent pairs).
    (a, b) -> (a cos - b sin, a sin + b cos)."""
    x = to64(x)
    a, b = x[..., 0::2], x[..., 1::2]
    c = to64(np.cos(ang))[None, :, None, :]
    s = to64(np.sin(ang))[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def attention(q, k, v):
    """softmax(q k^T / sqrt(dh)) v per (batch, head); q [B,nh,Nq,dh], k/v [B,nh,Nk,dh].
    The full score matrix, no mask (READING: a slice is denoised jointly)."""
    q, k, v = to64(q), to64(k), to64(v)
    s = q @ np.swapaxes(k, -1, -2) / math.sqrt(q.shape[-1])
    return softmax(s, axis=-1) @ v


def split_heads(x, nh):
    B, N, D = x.shape
    return x.reshape(B, N, nh, D // nh).transpose(0, 2, 1, 3)


def merge_heads(x):
    B, nh, N, dh = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, N, nh * dh)


def self_attention(h, Wb, ang, cfg, attn=attention, qkv_linear=linear):
    """QKV projection (``qkv_linear``), q/k RMSNorm (full width), 3-D rotary,
    softmax attention (``attn``: ``attention`` here, or the FP8 forms of
    oracle/mxfp8.py for both). Returns the head-merged output before the
    output projection, [B, N, D]."""
    D, nh = cfg.dim, cfg.n_heads
    qkv = qkv_linear(h, Wb["qkv.w"], Wb["qkv.b"])
    q, k, v = qkv[..., :D], qkv[..., D:2 * D], qkv[..., 2 * D:]
    q = rms_norm(q, Wb["norm_q.g"], cfg.eps)
    k = rms_norm(k, Wb["norm_k.g"], cfg.eps)
    B, N, _ = q.shape
    q = apply_rope(q.reshape(B, N, nh, -1), ang).reshape(B, N, D)
    k = apply_rope(k.reshape(B, N, nh, -1), ang).reshape(B, N, D)
    return merge_heads(attn(split_heads(q, nh), split_heads(k, nh), split_heads(v, nh)))


def audio_kv(audio, Wb, cfg):
    """Audio keys (RMSNorm'd) and values from the audio tokens [B, La, D]; no rotary."""
    D = cfg.dim
    kv = linear(audio, Wb["ckv.w"], Wb["ckv.b"])
    return rms_norm(kv[..., :D], Wb["norm_ck.g"], cfg.eps), kv[..., D:]


def cross_attention(h3, kc, vc, Wb, cfg):
    """Audio cross-attention, before its output projection, [B, N, D].

    The gizai:flashhead page (overview) organises audio as 5 latent frames of 32
    tokens. READING: a query token of latent frame f attends to the audio
    tokens of frame f only (cfg.cross_full=False); cross_full=True attends to
    all of them.
    """
    nh = cfg.n_heads
    qc = rms_norm(linear(h3, Wb["cq.w"], Wb["cq.b"]), Wb["norm_cq.g"], cfg.eps)
    qh, kh, vh = split_heads(qc, nh), split_heads(kc, nh), split_heads(vc, nh)
    if cfg.cross_full:
        return merge_heads(attention(qh, kh, vh))
    hw, apf = cfg.height * cfg.width, cfg.audio_per_frame
    out = np.empty_like(qh)
    for f in range(cfg.frames):
        qs, ks = slice(f * hw, (f + 1) * hw), slice(f * apf, (f + 1) * apf)
        out[:, :, qs] = attention(qh[:, :, qs], kh[:, :, ks], vh[:, :, ks])
    return merge_heads(out)


# ----------------------------------------------------------------------------
# block, forward, sampler
# ----------------------------------------------------------------------------
def block_weights(W, i):
    p = f"blocks.{i}."
    return {k[len(p):]: v for k, v in W.items() if k.startswith(p)}


def dit_block(x, e0, audio, Wb, cfg, ang, ffn_linear=linear, attn=attention, qkv_linear=linear):
    """One Wan-style block on the residual stream x [B, N, D].

    mods = table + e0 ([B, 6, D]): shift/scale/gate for self-attention, then
    for the FFN (READING of the order).
      x += gate_sa * O(SA(LN(x)(1+scale_sa)+shift_sa))
      x += CO(CA(LN_affine(x), audio))           (ungated)
      x += gate_ff * FFN(LN(x)(1+scale_ff)+shift_ff)

    ffn_linear is the product used for the FFN's two layers, attn the
    self-attention and qkv_linear its input projection: ``linear`` and
    ``attention`` here, or the block-scaled FP8 forms of oracle/mxfp8.py for
    the FP8 variants.
    """
    x = to64(x)
    m = to64(Wb["mod"])[None] + to64(e0)
    h = modulate(layer_norm(x, cfg.eps), m[:, 0], m[:, 1])
    x = x + m[:, 2][:, None, :] * linear(self_attention(h, Wb, ang, cfg, attn, qkv_linear), Wb["o.w"], Wb["o.b"])
    h3 = layer_norm(x, cfg.eps, Wb["norm3.g"], Wb["norm3.b"])
    kc, vc = audio_kv(audio, Wb, cfg)
    x = x + linear(cross_attention(h3, kc, vc, Wb, cfg), Wb["co.w"], Wb["co.b"])
    h = modulate(layer_norm(x, cfg.eps), m[:, 3], m[:, 4])
    u = gelu_tanh(ffn_linear(h, Wb["ffn1.w"], Wb["ffn1.b"]))
    return x + m[:, 5][:, None, :] * ffn_linear(u, Wb["ffn2.w"], Wb["ffn2.b"])


def dit_block_from_temb(x, e, audio, W, i, cfg, ffn_linear=linear, attn=attention, qkv_linear=linear):
    """Block i with its modulation derived from a time embedding e [B, D]:
    e0 = Linear(SiLU(e)) (the shared time projection)."""
    e0 = linear(silu(e), W["time_proj.w"], W["time_proj.b"]).reshape(-1, 6, cfg.dim)
    return dit_block(x, e0, audio, block_weights(W, i), cfg, rope_angles(cfg), ffn_linear, attn, qkv_linear)


def patchify(latent):
    """[B, C, F, H, W] -> tokens [B, F*H*W, C] in (f, r, c) order. A 1x1 patch:
    at 512x512 the LTX latent is already 16x16 per frame (gizai:flashhead page)."""
    B, C = latent.shape[:2]
    return np.moveaxis(to64(latent), 1, -1).reshape(B, -1, C)


def unpatchify(tokens, cfg):
    B = tokens.shape[0]
    t = to64(tokens).reshape(B, cfg.frames, cfg.height, cfg.width, -1)
    return np.moveaxis(t, -1, 1)


def dit_flow(latent, sigma, audio, W, cfg, blocks=None, ffn_linear=linear, attn=attention, qkv_linear=linear):
    """Flow prediction v [B, C, F, H, W] of the DiT at noise level sigma (scalar)."""
    B = latent.shape[0]
    e, e0 = time_embedding(np.full(B, sigma, dtype=np.float64), W, cfg)
    ang = rope_angles(cfg)
    x = linear(patchify(latent), W["patch.w"], W["patch.b"])
    for i in (range(cfg.n_blocks) if blocks is None else blocks):
        x = dit_block(x, e0, audio, block_weights(W, i), cfg, ang, ffn_linear, attn, qkv_linear)
    hm = to64(W["head.mod"])[None] + e[:, None, :]          # [B, 2, D]: shift, scale
    h = modulate(layer_norm(x, cfg.eps), hm[:, 0], hm[:, 1])
    return unpatchify(linear(h, W["head.w"], W["head.b"]), cfg)


def pin_motion(latent, motion):
    """The first Fm latent frames are the previous slice's motion (gizai:flashhead
    page, overview)."""
    out = to64(latent).copy()
    out[:, :, :motion.shape[2]] = to64(motion)
    return out


def euler_step(latent, v, sigma, sigma_next):
    """Flow-matching Euler update x <- x + (sigma' - sigma) v.

    READING: the configs' "4 flow-matching Euler steps"; the audio-cpp page's
    "Variant boundaries" names a re-noising update for distilled checkpoints
    without defining it; with the model's own noise estimate re-injected it is
    this same update (see tests).
    """
    return to64(latent) + (float(sigma_next) - float(sigma)) * to64(v)


def denoise_slice(noise, motion, audio, sigmas, W, cfg, ffn_linear=linear, attn=attention, qkv_linear=linear):
    """Noise latent [B,C,F,H,W] -> denoised latent after len(sigmas)-1 steps,
    the motion frames pinned before the first step and after every step."""
    x = pin_motion(noise, motion)
    for i in range(len(sigmas) - 1):
        v = dit_flow(x, sigmas[i], audio, W, cfg, ffn_linear=ffn_linear, attn=attn, qkv_linear=qkv_linear)
        x = pin_motion(euler_step(x, v, sigmas[i], sigmas[i + 1]), motion)
    return x


def rel_err(got, ref, motion_frames=0):
    """max|g - r| / max|r| over the non-motion latent frames (axis 2) when
    motion_frames > 0, else over everything."""
    g, r = to64(got), to64(ref)
    if motion_frames:
        g, r = g[:, :, motion_frames:], r[:, :, motion_frames:]
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-300))


def err_stats(got, ref, motion_frames=0):
    """The comparison metric and its two companions, over the same elements as
    rel_err: the max-norm error max|g - r| / max|r|, the relative L2 error
    ||g - r|| / ||r||, and the 99.9th percentile of |g - r| / max|r| (one
    outlier moves the first, not the other two)."""
    g, r = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if motion_frames:
        g, r = g[:, :, motion_frames:], r[:, :, motion_frames:]
    d, scale = np.abs(g - r), max(np.abs(r).max(), 1e-300)
    return {"max": float(d.max() / scale), "rel_l2": float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)),
            "p999": float(np.percentile(d, 99.9) / scale)}
