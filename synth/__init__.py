"""Seeded synthetic weights and inputs for the FlashHead Lite DiT slice denoiser.

This module is the one place both sides of a parity check draw their data from:
the CPU oracle (``oracle/``) and the HIP library (``audio_driven_talking_amd``).
It holds workload sizes, tensor names/shapes/dtypes and seeded random numbers,
and nothing of the method's arithmetic (no norms, no attention, no sampler).

Workloads follow the gizai:flashhead reference page (overview paragraph): a
512x512 picture coded to a latent of 5 frames of 16x16, 5 latent frames of 32
audio tokens, 30 blocks of width 1536 with 12 heads, 4 flow-matching steps.
The SoulX-FlashHead audio-cpp page (section "Generate") fixes 4 steps and seed
42 as defaults; its "Variant boundaries" section says the transformer's
dimensions come from an embedded configuration, hence every size below is a
plain runtime value.

Distributions (none is on the pages; they are stated here once):
  * matrices: N(0, 0.02) drawn in float32, rounded to bfloat16 (round to
    nearest even); both sides use exactly these values;
  * biases, modulation tables: N(0, 0.02), float32;
  * norm gains: 1 + N(0, 0.02), float32;
  * latent noise, motion latent, audio tokens, residual stream, time
    embedding, speech-encoder states: N(0, 1), float32.
Every tensor has its own generator, keyed by (seed, crc32(name)), so a subset
of blocks can be drawn without drawing the rest.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import os
import zlib

import numpy as np

WEIGHT_SEED = 1234
NOISE_SEED = 42
MOTION_SEED = 43
AUDIO_SEED = 44
RESID_SEED = 41
TEMB_SEED = 45
STATES_SEED = 46
LANE_SEED_STRIDE = 100


@dataclasses.dataclass(frozen=True)
class DiTConfig:
    """Sizes of one DiT and its slice latent (all plain values)."""
    n_blocks: int = 30
    dim: int = 1536
    n_heads: int = 12
    head_dim: int = 128
    ffn_dim: int = 8960
    in_ch: int = 16
    out_ch: int = 16
    frames: int = 5
    height: int = 16
    width: int = 16
    motion_frames: int = 2
    audio_per_frame: int = 32
    freq_dim: int = 256
    cross_full: bool = False   # False: frame-local audio attention; True: all audio tokens
    eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def tokens(self) -> int:
        return self.frames * self.height * self.width

    @property
    def audio_tokens(self) -> int:
        return self.frames * self.audio_per_frame

    def replace(self, **kw) -> "DiTConfig":
        return dataclasses.replace(self, **kw)


# The five workloads. Sizes only; seeds are the module constants above.
CONFIGS = {
    # 2 blocks, width 256, 2 heads x 128, FFN 1024; latent 2x8x8; 64 audio tokens; 1 step.
    "toy": DiTConfig(n_blocks=2, dim=256, n_heads=2, head_dim=128, ffn_dim=1024,
                     frames=2, height=8, width=8, motion_frames=1),
    # one real-shape block: 1280 tokens, width 1536, 12 heads, FFN 8960, 160 audio tokens
    "block": DiTConfig(n_blocks=1),
    # full Lite slice: 30 blocks, 5x16x16 latent, 2 motion frames, 4 steps
    "slice": DiTConfig(),
    # 768x768 output: latent 5x24x24 (2880 tokens)
    "slice768": DiTConfig(height=24, width=24),
}
TOY_SIGMAS = (1.0, 0.0)
SLICE_SIGMAS = (1.0, 0.75, 0.5, 0.25, 0.0)


def param_specs(cfg: DiTConfig, blocks=None):
    """(name, shape, kind) of every tensor, in blob order.

    kind is 'matrix' (bf16, stored [out, in]), 'vector' (f32) or 'gain' (f32).
    ``qkv.w`` stacks the q, k and v projections ([3D, D], rows q then k then v);
    ``ckv.w`` stacks the audio k and v projections ([2D, D]).
    ``mod`` is a block's modulation table [6, D]: rows shift, scale, gate of the
    self-attention branch, then shift, scale, gate of the FFN branch.
    ``head.mod`` is the output norm's table [2, D]: rows shift, scale.
    """
    D, Fd, C, Co, Fq = cfg.dim, cfg.ffn_dim, cfg.in_ch, cfg.out_ch, cfg.freq_dim
    specs = [
        ("time_in.w", (D, Fq), "matrix"), ("time_in.b", (D,), "vector"),
        ("time_out.w", (D, D), "matrix"), ("time_out.b", (D,), "vector"),
        ("time_proj.w", (6 * D, D), "matrix"), ("time_proj.b", (6 * D,), "vector"),
        ("patch.w", (D, C), "matrix"), ("patch.b", (D,), "vector"),
        ("head.w", (Co, D), "matrix"), ("head.b", (Co,), "vector"),
        ("head.mod", (2, D), "vector"),
    ]
    ids = range(cfg.n_blocks) if blocks is None else blocks
    for i in ids:
        p = f"blocks.{i}."
        specs += [
            (p + "mod", (6, D), "vector"),
            (p + "qkv.w", (3 * D, D), "matrix"), (p + "qkv.b", (3 * D,), "vector"),
            (p + "norm_q.g", (D,), "gain"), (p + "norm_k.g", (D,), "gain"),
            (p + "o.w", (D, D), "matrix"), (p + "o.b", (D,), "vector"),
            (p + "norm3.g", (D,), "gain"), (p + "norm3.b", (D,), "vector"),
            (p + "cq.w", (D, D), "matrix"), (p + "cq.b", (D,), "vector"),
            (p + "ckv.w", (2 * D, D), "matrix"), (p + "ckv.b", (2 * D,), "vector"),
            (p + "norm_cq.g", (D,), "gain"), (p + "norm_ck.g", (D,), "gain"),
            (p + "co.w", (D, D), "matrix"), (p + "co.b", (D,), "vector"),
            (p + "ffn1.w", (Fd, D), "matrix"), (p + "ffn1.b", (Fd,), "vector"),
            (p + "ffn2.w", (D, Fd), "matrix"), (p + "ffn2.b", (D,), "vector"),
        ]
    return specs


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([seed, zlib.crc32(name.encode())])


def _draw(seed, name, shape, kind):
    g = _rng(seed, name)
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    if kind == "matrix":
        return bf16_bits(x)                      # uint16 bf16 bits
    if kind == "gain":
        return (x + np.float32(1.0)).astype(np.float32)
    return x.astype(np.float32)


def make_weights(cfg: DiTConfig, seed: int = WEIGHT_SEED, blocks=None, threads=None):
    """dict name -> array. Matrices come as uint16 bf16 bits, the rest as float32."""
    specs = param_specs(cfg, blocks)
    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(threads) as ex:
        arrs = list(ex.map(lambda s: _draw(seed, *s), specs))
    return {s[0]: a for s, a in zip(specs, arrs)}


def weights_f32(weights: dict) -> dict:
    """The same weights with every matrix widened to float32 values (exact)."""
    return {k: (bf16_to_f32(v) if v.dtype == np.uint16 else v) for k, v in weights.items()}


def weights_digest(weights: dict) -> str:
    h = hashlib.sha256()
    for k in sorted(weights):
        h.update(k.encode())
        h.update(np.ascontiguousarray(weights[k]).tobytes())
    return h.hexdigest()


def normal(shape, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def slice_inputs(cfg: DiTConfig, batch: int = 1):
    """Noise latent [B,C,F,H,W], motion latent [B,C,Fm,H,W], audio tokens [B,La,D].

    Lane b draws from seeds (42, 43, 44) + 100*b, so lane b of a batch equals
    the single-lane inputs of that lane.
    """
    C, F, H, W, Fm = cfg.in_ch, cfg.frames, cfg.height, cfg.width, cfg.motion_frames
    lat = np.stack([normal((C, F, H, W), NOISE_SEED + LANE_SEED_STRIDE * b) for b in range(batch)])
    mot = np.stack([normal((C, Fm, H, W), MOTION_SEED + LANE_SEED_STRIDE * b) for b in range(batch)])
    aud = np.stack([normal((cfg.audio_tokens, cfg.dim), AUDIO_SEED + LANE_SEED_STRIDE * b)
                    for b in range(batch)])
    return lat, mot, aud


def block_inputs(cfg: DiTConfig, batch: int = 1):
    """Residual stream x [B,N,D], time embedding e [B,D], audio tokens [B,La,D]."""
    x = np.stack([normal((cfg.tokens, cfg.dim), RESID_SEED + LANE_SEED_STRIDE * b) for b in range(batch)])
    e = np.stack([normal((cfg.dim,), TEMB_SEED + LANE_SEED_STRIDE * b) for b in range(batch)])
    a = np.stack([normal((cfg.audio_tokens, cfg.dim), AUDIO_SEED + LANE_SEED_STRIDE * b)
                  for b in range(batch)])
    return x, e, a


# ---------------------------------------------------------------- audio projection front end
@dataclasses.dataclass(frozen=True)
class AudioProjConfig:
    """Sizes of the audio projection (speech-encoder states -> audio tokens).

    The gizai:flashhead page fixes 12 layers' states at 200 frames, 5 states
    around each of 33 frames, 5 latent frames of 32 tokens; channels 768 is the
    width of wav2vec 2.0 base; the hidden width is not on the pages (a plain
    choice)."""
    layers: int = 12
    state_frames: int = 200
    channels: int = 768
    window: int = 5
    video_frames: int = 33
    temporal_stride: int = 8
    hidden: int = 512
    tokens: int = 32
    dim: int = 1536
    eps: float = 1e-6

    @property
    def latent_frames(self) -> int:
        return 1 + (self.video_frames - 1) // self.temporal_stride

    @property
    def feat(self) -> int:
        return self.window * self.layers * self.channels

    def replace(self, **kw) -> "AudioProjConfig":
        return dataclasses.replace(self, **kw)


AUDIO_CONFIGS = {
    # matches the toy DiT: 2 latent frames x 32 tokens of width 256
    "toy": AudioProjConfig(layers=2, state_frames=40, channels=64, video_frames=9, hidden=128, dim=256),
    # the Lite slice: 5 latent frames x 32 tokens of width 1536
    "lite": AudioProjConfig(),
}


def audio_param_specs(acfg: AudioProjConfig):
    """(name, shape, kind) of the audio projection's tensors, in blob order."""
    F, P, TD, D = acfg.feat, acfg.hidden, acfg.tokens * acfg.dim, acfg.dim
    return [
        ("proj1.w", (P, F), "matrix"), ("proj1.b", (P,), "vector"),
        ("proj1vf.w", (P, F), "matrix"), ("proj1vf.b", (P,), "vector"),
        ("proj2.w", (P, P), "matrix"), ("proj2.b", (P,), "vector"),
        ("proj3.w", (TD, P), "matrix"), ("proj3.b", (TD,), "vector"),
        ("projNorm.g", (D,), "gain"), ("projNorm.b", (D,), "vector"),
    ]


def make_audio_weights(acfg: AudioProjConfig, seed: int = WEIGHT_SEED):
    """dict name -> array, drawn as make_weights draws the DiT's."""
    return {n: _draw(seed, n, shape, kind) for n, shape, kind in audio_param_specs(acfg)}


def audio_states(acfg: AudioProjConfig, batch: int = 1):
    """Speech-encoder states [B, layers, state_frames, channels], N(0, 1); lane b
    draws from seed 46 + 100 b."""
    return np.stack([normal((acfg.layers, acfg.state_frames, acfg.channels), STATES_SEED + LANE_SEED_STRIDE * b)
                     for b in range(batch)])


# ---------------------------------------------------------------- colour match
COLOR_SEED = 47
# (frames, height, width, picture height, picture width): the Lite slice decodes
# 33 frames of 512 x 512 and matches them to the 512 x 512 picture (gizai:flashhead
# reference page, overview paragraph and FlashHead.picture)
COLOR_SHAPES = {"toy": (5, 24, 40, 32, 20), "ragged": (3, 7, 9, 5, 11), "slice": (33, 512, 512, 512, 512)}


def _color_field(rng, h, w):
    """A smooth [3, h, w] colour field in about [0.1, 0.9]: a few low-frequency
    cosines per channel on the unit square, so fields drawn at other sizes
    from the same generator state look alike."""
    y, x = np.meshgrid(np.linspace(0.0, 1.0, h), np.linspace(0.0, 1.0, w), indexing="ij")
    out = np.empty((3, h, w))
    for c in range(3):
        f = np.full((h, w), 0.5)
        for _ in range(4):
            ky, kx, ph, amp = rng.uniform(0.5, 4.0), rng.uniform(0.5, 4.0), rng.uniform(0, 2 * np.pi), 0.1
            f += amp * np.cos(2 * np.pi * (ky * y + kx * x) + ph)
        out[c] = f
    return out


def color_inputs(n_frames, height, width, ref_height, ref_width, seed: int = COLOR_SEED):
    """Decoded frames [3, F, H, W] and the picture [3, H', W'], float32 sRGB
    values in [0, 1].

    Recipe (not on the pages; stated once here): the picture is a smooth
    colour field; frame f is the same field drawn at the frames' size, with a
    per-frame, per-channel gain U(0.8, 1.2) and offset U(-0.1, 0.1) (a colour
    cast for the correction to remove) and N(0, 0.02) noise, clipped to
    [0, 1], so bright and dark corners saturate exactly at 0 and 1.
    """
    rng = np.random.default_rng([seed, n_frames, height, width, ref_height, ref_width])
    state = rng.bit_generator.state
    pic = np.clip(_color_field(rng, ref_height, ref_width), 0.0, 1.0)
    rng.bit_generator.state = state
    base = _color_field(rng, height, width)
    gain = rng.uniform(0.8, 1.2, (3, n_frames, 1, 1))
    off = rng.uniform(-0.1, 0.1, (3, n_frames, 1, 1))
    frames = base[:, None] * gain + off + rng.normal(0.0, 0.02, (3, n_frames, height, width))
    return np.clip(frames, 0.0, 1.0).astype(np.float32), pic.astype(np.float32)


# ---------------------------------------------------------------- video VAE decoder
VAE_LATENT_SEED = 48


@dataclasses.dataclass(frozen=True)
class VaeConfig:
    """Sizes of the video decoder that turns a slice latent into frames.

    The pages fix the latent (the gizai:flashhead page, overview paragraph:
    5 frames of 16 x 16 for a 512 x 512 picture, 33 decoded frames) and the
    strides (the toolkit page: LTX stride 32 in space; 33 = 1 + 4 x 8 frames
    from 5 latent frames, stride 8 in time). The layer widths are not on the
    pages: `widths` are the decoder's channel counts at its four resolutions
    (latent, x2, x4, x8 in space), a plain choice; `patch` is the last
    depth-to-space step (4 x 4 pixels per position)."""
    latent_ch: int = 16
    frames: int = 5
    height: int = 16
    width: int = 16
    widths: tuple = (256, 128, 64, 32)
    out_ch: int = 3
    patch: int = 4
    eps: float = 1e-6

    @property
    def out_frames(self) -> int:
        return 8 * (self.frames - 1) + 1

    @property
    def out_height(self) -> int:
        return self.height * 8 * self.patch

    @property
    def out_width(self) -> int:
        return self.width * 8 * self.patch

    def replace(self, **kw) -> "VaeConfig":
        return dataclasses.replace(self, **kw)


VAE_CONFIGS = {
    # small widths, a 2-frame 4 x 4 latent: 9 frames of 128 x 128
    "toy": VaeConfig(frames=2, height=4, width=4, widths=(64, 32, 32, 32)),
    # a 3-frame 6 x 10 latent (180 positions: ragged tiles): 17 frames of 192 x 320
    "ragged": VaeConfig(frames=3, height=6, width=10, widths=(128, 64, 32, 32)),
    # a 5-frame 3 x 64 latent, narrow: the up-sampling into stage 2 runs on frames of
    # 6 x 128 positions (two 4-row tiles, the second half empty) -> 33 frames of 96 x 2048
    "ragged_h": VaeConfig(frames=5, height=3, width=64, widths=(32, 32, 32, 32)),
    # the Lite slice: 5 x 16 x 16 latent -> 33 frames of 512 x 512
    "slice": VaeConfig(),
}


def vae_param_specs(vcfg: VaeConfig):
    """(name, shape, kind) of the decoder's tensors, in blob order. Convolution
    kernels are [C_out, 3, 3, 3, C_in] (time, row, column taps, input channel
    fastest); the up-sampling convolutions have 8 C' outputs, ordered
    (sub-position, channel): output channel s C' + c fills sub-position s of
    the 2 x 2 x 2 block of channel c; conv_out has out_ch patch^2 outputs,
    ordered (colour, row, column) of the patch."""
    w, P = vcfg.widths, vcfg.patch
    specs = [("conv_in.w", (w[0], 3, 3, 3, vcfg.latent_ch), "conv"), ("conv_in.b", (w[0],), "vector")]
    for i in range(3):
        p = f"up{i}."
        specs += [(p + "norm1.g", (w[i],), "gain"), (p + "conv1.w", (w[i], 3, 3, 3, w[i]), "conv"),
                  (p + "conv1.b", (w[i],), "vector"), (p + "norm2.g", (w[i],), "gain"),
                  (p + "conv2.w", (w[i], 3, 3, 3, w[i]), "conv"), (p + "conv2.b", (w[i],), "vector"),
                  (p + "up.w", (8 * w[i + 1], 3, 3, 3, w[i]), "conv"), (p + "up.b", (8 * w[i + 1],), "vector")]
    specs += [("norm_out.g", (w[3],), "gain"), ("conv_out.w", (vcfg.out_ch * P * P, 3, 3, 3, w[3]), "conv"),
              ("conv_out.b", (vcfg.out_ch * P * P,), "vector")]
    return specs


def f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bits (round to nearest even), as uint16."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def make_vae_weights(vcfg: VaeConfig, seed: int = WEIGHT_SEED):
    """dict name -> array: convolution kernels as uint16 float16 bits drawn
    N(0, 1) / sqrt(27 C_in) in float32 (unit gain through a 3 x 3 x 3
    convolution of unit-RMS inputs); biases N(0, 0.02) and norm gains
    1 + N(0, 0.02) as float32."""
    out = {}
    for name, shape, kind in vae_param_specs(vcfg):
        if kind == "conv":
            g = _rng(seed, name)
            fan_in = 27 * shape[-1]
            x = g.standard_normal(shape, dtype=np.float32) / np.float32(np.sqrt(fan_in))
            out[name] = f16_bits(x)
        else:
            out[name] = _draw(seed, name, shape, kind)
    return out


def vae_weights_f32(weights: dict) -> dict:
    """The decoder weights with the float16 kernels widened to float32 (exact)."""
    return {k: (f16_to_f32(v) if v.dtype == np.uint16 else v) for k, v in weights.items()}


def vae_latent(vcfg: VaeConfig, seed: int = VAE_LATENT_SEED):
    """A denoised slice latent [latent_ch, frames, height, width], N(0, 1) float32."""
    return normal((vcfg.latent_ch, vcfg.frames, vcfg.height, vcfg.width), seed)
