"""Float64 oracle of the video decoder after the denoiser (slice latent ->
33 RGB frames), an assumed LTX-style layout.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * gizai:flashhead reference page, overview paragraph: LTX-Video 0.9's VAE
    codes the 512 x 512 picture to a latent of 5 frames of 16 x 16, and after
    the denoise "the VAE decodes 33 frames", whose colours are then matched
    to the picture's;
  * toolkit page "SoulX-FlashHead -- Talking Head Video Generation": Lite
    uses the LTX-Video VAE with spatial stride 32;
  * audio-cpp page "SoulX-FlashHead", section "Variant boundaries": the Lite
    VAE's convolutions (Conv3D) take F16 operands with F32 accumulation and
    F16 output storage, the channel bias added in F32 to the F16 convolution
    result before the final F16 cast; residual storage is F16; normalisation
    accumulates in F32 with F16 output; the VAE's public inputs and outputs
    are F32.

The layers themselves are not on the pages. READINGS (an assumed layout in
the shape of a causal video VAE decoder; each is the plainest choice the
fixed facts allow):
  V1 every convolution is 3 x 3 x 3, stride 1; time is padded causally (two
     copies of the first frame before it, nothing after), space with one
     zero on each side;
  V2 the decoder is conv_in (latent channels -> widths[0]), then three
     stages, each a residual block (RMS norm over channels with a gain,
     SiLU, convolution, twice, added to the block's input) and an
     up-sampling convolution to 8 widths[i+1] channels followed by depth to
     space (2 x 2 x 2) that drops the first of the doubled frames (so 5 -> 9
     -> 17 -> 33 frames and 16 -> 128 in space), then RMS norm, SiLU and
     conv_out to 3 x 4 x 4 channels unfolded into 4 x 4 pixels (512 x 512);
  V3 channel orders: up-sampling output channel s C' + c (s = 4 dt + 2 dh + dw)
     goes to sub-position (dt, dh, dw) of channel c; conv_out channel
     c 16 + 4 ph + pw goes to pixel (4 h + ph, 4 w + pw) of colour c;
  V4 the RMS norm is x / sqrt(mean over channels of x^2 + eps) * g, eps 1e-6,
     and the SiLU is applied to its output before the one F16 store;
  V5 the decoder's output v in [-1, 1] becomes frames (v + 1) / 2 clamped to
     [0, 1] (float32 RGB planes, the colour match's input);
  V6 numerics as the audio-cpp page states them: every stored activation is
     rounded to F16 (round to nearest even) -- the latent as the first
     convolution's operand, each convolution's sum before and after its
     bias, each norm + SiLU output, each residual sum -- while sums run here
     in float64 (at least the F32 the page names). ``half=False`` keeps every
     value in float64 (the exact function, used by the pins).
"""
from __future__ import annotations

import numpy as np

__all__ = ["f16", "conv3d", "norm_silu", "res_block", "upsample", "unpatchify", "decode", "to_frames"]


def f16(x):
    """Round to IEEE binary16 (round to nearest even) and back to float64 (V6)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def conv3d(x, w, b, half=True):
    """x [C_in, T, H, W], w [C_out, 3, 3, 3, C_in], b [C_out] -> [C_out, T, H, W].

    out[o, t, h, w] = sum over taps (a, p, q) and input channels i of
    w[o, a, p, q, i] * xp[i, t + a, h + p, w + q], xp being x with two copies
    of frame 0 before it (causal, V1) and a zero border of one in space. With
    half: F16 operands, the sum rounded to F16, the bias added, rounded again
    (the audio-cpp page's Variant boundaries)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if half:
        x, w = f16(x), f16(w)
    C, T, H, W = x.shape
    xp = np.concatenate([x[:, :1], x[:, :1], x], axis=1)
    xp = np.pad(xp, ((0, 0), (0, 0), (1, 1), (1, 1)))
    out = np.zeros((w.shape[0], T, H, W))
    for a in range(3):
        for p in range(3):
            for q in range(3):
                out += np.tensordot(w[:, a, p, q, :], xp[:, a:a + T, p:p + H, q:q + W], axes=([1], [0]))
    bias = np.asarray(b, dtype=np.float64)[:, None, None, None]
    if half:
        return f16(f16(out) + bias)
    return out + bias


def norm_silu(x, g, eps, half=True):
    """RMS norm over the channel axis with gain g (V4), then SiLU; one F16 store."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt((x * x).mean(axis=0, keepdims=True) + eps) * np.asarray(g, dtype=np.float64)[:, None, None, None]
    y = y / (1.0 + np.exp(-y))
    return f16(y) if half else y


def res_block(x, W, p, eps, half=True):
    """x + conv2(norm_silu(conv1(norm_silu(x)))) with the block's tensors
    named p + {norm1.g, conv1.w, conv1.b, norm2.g, conv2.w, conv2.b}; the sum
    stored in F16 (residual storage, V6)."""
    h = conv3d(norm_silu(x, W[p + "norm1.g"], eps, half), W[p + "conv1.w"], W[p + "conv1.b"], half)
    h = conv3d(norm_silu(h, W[p + "norm2.g"], eps, half), W[p + "conv2.w"], W[p + "conv2.b"], half)
    s = np.asarray(x, dtype=np.float64) + h
    return f16(s) if half else s


def upsample(x, w, b, half=True):
    """Convolution to 8 C' channels, then depth to space (V3): channel s C' + c,
    s = 4 dt + 2 dh + dw, at (t, h, w) goes to (2 t + dt, 2 h + dh, 2 w + dw)
    of channel c; the first of the 2T frames is dropped (V2)."""
    y = conv3d(x, w, b, half)
    C8, T, H, W = y.shape
    c = C8 // 8
    z = y.reshape(2, 2, 2, c, T, H, W).transpose(3, 4, 0, 5, 1, 6, 2).reshape(c, 2 * T, 2 * H, 2 * W)
    return z[:, 1:]


def unpatchify(y, out_ch, patch):
    """[out_ch patch^2, T, H, W] -> [out_ch, T, H patch, W patch]: channel
    c patch^2 + ph patch + pw is pixel (h patch + ph, w patch + pw) of colour c (V3)."""
    _, T, H, W = y.shape
    return y.reshape(out_ch, patch, patch, T, H, W).transpose(0, 3, 4, 1, 5, 2).reshape(out_ch, T, H * patch,
                                                                                      W * patch)


def to_frames(v):
    """Decoder output in [-1, 1] -> RGB values in [0, 1] (V5)."""
    return np.clip((np.asarray(v, dtype=np.float64) + 1.0) * 0.5, 0.0, 1.0)


def decode(latent, W, vcfg, half=True):
    """Slice latent [latent_ch, F, H, W] -> frames [out_ch, 8 (F - 1) + 1, 32 H, 32 W]
    in [0, 1] (V1-V6)."""
    x = conv3d(latent, W["conv_in.w"], W["conv_in.b"], half)
    for i in range(3):
        x = res_block(x, W, f"up{i}.", vcfg.eps, half)
        x = upsample(x, W[f"up{i}.up.w"], W[f"up{i}.up.b"], half)
    y = conv3d(norm_silu(x, W["norm_out.g"], vcfg.eps, half), W["conv_out.w"], W["conv_out.b"], half)
    return to_frames(unpatchify(y, vcfg.out_ch, vcfg.patch))
