"""Oracle of the block-scaled FP8 (MX) quantisation of GEMM operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: the page "SoulX-LiveAct, real-time human animation video
from audio and a still image" (section "The three contributions, and what
each one buys you", and the installation section) attributes the sibling
system's real-time speed to end-to-end adaptive FP8 precision, with FP8 GEMM
and FP8 attention kernels; the FlashHead pages name no number format for the
DiT beyond bf16/F32 (and a Q8 weight package). The FP8 path here is
therefore an option of this library, checked against the same float64
oracle at a looser bound, with the quantiser itself pinned.

READING (the MX convention of the OCP Microscaling format, which gfx950's
scaled MFMA implements): a row is cut into blocks of 32 consecutive elements
along K; a block with max |x| = a > 0 gets the power-of-two scale
X = 2^(floor(log2 a) - 8) (8 = the exponent of e4m3's largest power of two,
448 = 1.75 * 2^8), stored as the E8M0 byte floor(log2 a) - 8 + 127; each
element is x / X rounded to the nearest e4m3 value (ties to even), clamped
to +-448 first (x / X < 512 can exceed 448). An all-zero block gets X = 1.
e4m3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals
m/8 * 2^-6; no infinities; S.1111.111 is NaN (never produced here).

mx_linear is the FFN product of the FP8 variants of the block
(``dit_block(..., ffn_linear=mx_linear)``) and mx_attention their
self-attention (``attn=mx_attention``).

Decisions are taken on float32 inputs in float32-exact arithmetic (a power-
of-two division and a rounding on a power-of-two grid are exact in float64),
as the GPU takes them, so both sides produce the same codes.
"""
from __future__ import annotations

import numpy as np

from .dit import linear, to64

__all__ = ["BLOCK", "e4m3_decode", "e4m3_encode", "mx_quantize", "mx_dequantize", "mx_linear",
           "mx_attention"]

BLOCK = 32
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """e4m3 (FN) bytes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def e4m3_encode(q):
    """Round float values (|q| <= 448) to the nearest e4m3 code, ties to even."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    if np.any(a > E4M3_MAX):
        raise ValueError("e4m3_encode expects values clamped to +-448")
    # grid step: 2^(E - 3) for normal |q| in [2^E, 2^(E+1)), E >= -6; 2^-9 below 2^-6
    E = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    E = np.maximum(E, -6.0)
    step = 2.0 ** (E - 3)
    k = np.rint(a / step)                      # ties to even (the grid is uniform in the binade)
    mag = k * step                              # exact; may carry into the next binade (k = 16)
    # encode mag: exponent field and mantissa
    Em = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    sub = mag < 2.0 ** -6
    ef = np.where(sub, 0, Em + 7).astype(np.int64)
    mf = np.where(sub, mag / 2.0 ** -9, (mag / 2.0 ** Em - 1.0) * 8.0)
    mf = np.rint(mf).astype(np.int64)
    code = (ef << 3) | mf
    code = np.where(mag == 0, 0, code)
    return (code | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)  # the sign survives rounding to 0


def mx_quantize(x):
    """float32 array [..., K] (K a multiple of 32) -> (codes uint8 [..., K],
    scales uint8 [..., K/32]) by the rule above."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(*x.shape[:-1], K // BLOCK, BLOCK)
    amax = np.abs(xb).max(-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))   # amax = f * 2^ex, f in [0.5, 1)
    shared = np.where(amax > 0, ex - 1 - 8, 0)
    shared = np.clip(shared, -127, 127)
    q = np.clip(xb / (2.0 ** shared)[..., None], -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(q).reshape(x.shape)
    return codes, (shared + 127).astype(np.uint8)


def mx_dequantize(codes, scales):
    """Inverse map: codes [..., K] and E8M0 scales [..., K/32] -> float64."""
    v = e4m3_decode(codes)
    K = v.shape[-1]
    s = 2.0 ** (np.asarray(scales, dtype=np.float64) - 127.0)
    return (v.reshape(*v.shape[:-1], K // BLOCK, BLOCK) * s[..., None]).reshape(v.shape)


def mx_linear(x, w, b=None):
    """y = Q(x) Q(W)^T + b: both operands MX-quantised along their shared
    K axis (x's rows and W's rows, W stored [out, in]) from float32 values,
    then the product of the decoded values and the bias add in float64.

    This is the FP8 GEMM's arithmetic with exact accumulation: the hardware's
    scaled product sums the same decoded values (each code times its block's
    power of two) in float32.
    """
    xq = mx_dequantize(*mx_quantize(np.asarray(x, dtype=np.float64).astype(np.float32)))
    wq = mx_dequantize(*mx_quantize(np.asarray(w, dtype=np.float64).astype(np.float32)))
    return linear(xq, wq, b)


def _mx_round(x):
    """MX-FP8 round trip of float values along the last axis (float32 decisions)."""
    return mx_dequantize(*mx_quantize(np.asarray(x, dtype=np.float64).astype(np.float32)))


def mx_attention(q, k, v):
    """Softmax attention on MX-FP8 operands, q/k/v [B, nh, N, dh].

    READING (the page that names FP8 attention does not define it): each
    product's operands are quantised along that product's contraction axis,
    as in mx_linear -- q and k along dh for the scores; for the weighted sum
    the values along the keys (per output dimension) and the probabilities
    p = exp(s - max_j s) along the keys (per query); the sum in the
    denominator is of the unquantised p. So
        out = Q(p) Q(v) / sum_j p,   s = Q(q) Q(k)^T / sqrt(dh).
    """
    q, k, v = to64(q), to64(k), to64(v)
    s = _mx_round(q) @ np.swapaxes(_mx_round(k), -1, -2) / np.sqrt(q.shape[-1])
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    vq = np.swapaxes(_mx_round(np.swapaxes(v, -1, -2)), -1, -2)
    return (_mx_round(p) @ vq) / p.sum(axis=-1, keepdims=True)
