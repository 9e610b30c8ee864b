"""Pins of the MX-FP8 quantiser oracle (oracle/mxfp8.py) against what the e4m3
and MX definitions fix: every code decodes to its defining value, the encoder
is the nearest-value (ties-to-even) rounding found by brute force over all
codes, scales are powers of two that put the block maximum in [256, 512),
and the round trip stays within half a grid step."""
import numpy as np
import pytest

from oracle import mxfp8 as Q


def all_finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_decode_matches_the_format_definition():
    v = Q.e4m3_decode(all_finite_codes())
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    assert Q.e4m3_decode([0x38])[0] == 1.0 and Q.e4m3_decode([0x01])[0] == 2.0 ** -9  # 1.0, min subnormal
    assert Q.e4m3_decode([0x08])[0] == 2.0 ** -6 and Q.e4m3_decode([0x7E])[0] == 448.0
    assert np.isnan(Q.e4m3_decode([0x7F, 0xFF])).all()
    pos = np.sort(Q.e4m3_decode(np.arange(0, 0x7F)))
    assert np.all(np.diff(pos) > 0)                       # 127 distinct non-negative values
    assert len(np.unique(v)) == 253                       # +-0 collapse: 254 codes -> 253 values


def test_encoder_is_nearest_even_by_brute_force():
    grid = Q.e4m3_decode(np.arange(0, 0x7F))           # 0 .. 448, ascending
    codes = np.arange(0, 0x7F)
    rng = np.random.default_rng(0)
    q = np.concatenate([rng.uniform(0, 448, 20000), rng.uniform(0, 2.0 ** -5, 5000),
                        (grid[1:] + grid[:-1]) / 2])       # include every midpoint (ties)
    got = Q.e4m3_encode(q)
    d = np.abs(q[:, None] - grid[None, :])
    best = d.min(1, keepdims=True)
    cand = np.where(d == best, codes[None, :], 999)
    # ties go to the even mantissa (code's lowest bit 0)
    tie = (d == best).sum(1) > 1
    ref = np.where(tie, np.where(cand % 2 == 0, cand, 999).min(1), cand.min(1))
    np.testing.assert_array_equal(got, ref.astype(np.uint8))
    np.testing.assert_array_equal(Q.e4m3_encode(-q), ref.astype(np.uint8) | 0x80)  # sign bit only
    np.testing.assert_array_equal(Q.e4m3_encode([0.0, -0.0, -2.0 ** -12]), [0x00, 0x80, 0x80])  # signed zeros


def test_scales_put_block_max_in_range_and_round_trip_is_half_a_step():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    x[3, :32] = 0.0                                         # an all-zero block
    codes, scales = Q.mx_quantize(x)
    assert codes.shape == x.shape and scales.shape == (64, 8)
    amax = np.abs(x.reshape(64, 8, 32)).max(-1)
    X = 2.0 ** (scales.astype(np.float64) - 127)
    nz = amax > 0
    assert np.all((amax[nz] / X[nz] >= 256) & (amax[nz] / X[nz] < 512))
    assert scales[3, 0] == 127 and np.all(codes[3, :32] == 0)
    y = Q.mx_dequantize(codes, scales)
    xb, yb = x.reshape(64, 8, 32).astype(np.float64), y.reshape(64, 8, 32)
    # error <= half a step of the element's own binade (2^-4 relative) or of the subnormal grid,
    # except saturated elements (clamped to 448 X)
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(xb) / X[..., None], 1e-300))) - 3), 2.0 ** -9)
    sat = np.abs(xb) / X[..., None] > 448
    err = np.abs(xb - yb) / X[..., None]
    assert np.all(err[~sat] <= step[~sat] / 2 * (1 + 1e-12))
    assert np.all(np.abs(yb[sat]) == 448 * np.broadcast_to(X[..., None], xb.shape)[sat])


def test_scaled_dot_products_track_exact_ones():
    """A product of MX-quantised operands (the FP8 GEMM's arithmetic) is within a few
    percent of the exact product for random data: the bound the slices are held to."""
    rng = np.random.default_rng(2)
    a = rng.standard_normal((64, 1536)).astype(np.float32)
    w = (rng.standard_normal((96, 1536)) * 0.02).astype(np.float32)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    got = Q.mx_dequantize(*Q.mx_quantize(a)) @ Q.mx_dequantize(*Q.mx_quantize(w)).T
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel < 0.05


def _representable(rng, rows, K):
    """float32 [rows, K] whose every 32-block is e4m3 codes times one power of
    two, the block maximum a full-range code (so MX quantisation is the
    identity), with block scales spread over 2^-40 .. 2^40 along K and rows."""
    codes = rng.integers(0, 0x7E, (rows, K)).astype(np.uint8)
    codes = codes | (rng.integers(0, 2, (rows, K)).astype(np.uint8) << 7)
    codes[:, ::32] = 0x7E | (codes[:, ::32] & 0x80)          # |max| = 448 in every block
    v = Q.e4m3_decode(codes).reshape(rows, K // 32, 32)
    e = rng.integers(-40, 40, (rows, K // 32))
    return (v * 2.0 ** e[..., None]).reshape(rows, K).astype(np.float32)


def test_mx_linear_is_exact_on_representable_operands():
    """Quantisation must act along K on both operands: the blocks of x's rows
    and W's rows are representable there (and only there: along any other
    axis their scales, 2^80 apart, would flush the small values)."""
    rng = np.random.default_rng(3)
    x = _representable(rng, 24, 256)
    w = _representable(rng, 64, 256)
    b = rng.standard_normal(64)
    np.testing.assert_array_equal(Q.mx_dequantize(*Q.mx_quantize(x)), x)  # identity on the grid
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b
    np.testing.assert_array_equal(Q.mx_linear(x, w, b), ref)
    # the same operands blocked along the other axis are not representable
    wt = Q.mx_dequantize(*Q.mx_quantize(np.ascontiguousarray(w.T))).T
    assert not np.array_equal(wt, w)


def test_mx_linear_error_within_the_elementwise_bound():
    """|Q(x)Q(W)^T - x W^T| <= |x| e_W^T + e_x |W|^T + e_x e_W^T, with the element
    bound e = max(2^-4 |v|, 2^-10 X) (half a step, normal or subnormal grid),
    X = 2^(floor(log2 amax) - 8) from the block maximum, and 2^-3 |v| for
    elements above 448 X (saturation)."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((32, 512)) * np.exp(rng.uniform(-4, 4, (32, 512)))).astype(np.float32)
    w = (rng.standard_normal((48, 512)) * 0.03).astype(np.float32)

    def bound(v):
        v = v.astype(np.float64)
        vb = np.abs(v).reshape(v.shape[0], -1, 32)
        X = 2.0 ** (np.floor(np.log2(vb.max(-1))) - 8)[..., None]
        e = np.maximum(2.0 ** -4 * vb, 2.0 ** -10 * X)
        e = np.where(vb > 448 * X, 2.0 ** -3 * vb, e)
        return e.reshape(v.shape)

    ex, ew = bound(x), bound(w)
    ax, aw = np.abs(x.astype(np.float64)), np.abs(w.astype(np.float64))
    lim = ax @ ew.T + ex @ aw.T + ex @ ew.T
    err = np.abs(Q.mx_linear(x, w) - x.astype(np.float64) @ w.astype(np.float64).T)
    assert np.all(err <= lim * (1 + 1e-9))
    assert err.max() > 0                                     # it does quantise


def test_block_routes_both_ffn_layers_through_the_product_hook():
    import oracle as O
    from synth import CONFIGS, make_weights, weights_f32, block_inputs
    cfg = CONFIGS["toy"]
    W = weights_f32(make_weights(cfg))
    x, e, a = block_inputs(cfg, 1)
    seen = []

    def spy(h, w, b):
        seen.append((h.shape[-1], w.shape))
        return O.linear(h, w, b)

    ref = O.dit_block_from_temb(x, e, a, W, 0, cfg)
    got = O.dit_block_from_temb(x, e, a, W, 0, cfg, ffn_linear=spy)
    np.testing.assert_array_equal(got, ref)
    F = W["blocks.0.ffn1.w"].shape[0]
    assert seen == [(cfg.dim, (F, cfg.dim)), (F, (cfg.dim, F))]


def test_mx_attention_uniform_scores_average_the_quantised_values():
    """q = 0: every score is 0, p = 1 (exactly representable), so the output is
    the mean over keys of the values quantised along the keys."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, 2, 64, 32)) * np.exp(rng.uniform(-3, 3, (1, 2, 64, 1)))
    q = np.zeros((1, 2, 8, 32))
    k = rng.standard_normal((1, 2, 64, 32))
    vq = np.swapaxes(Q.mx_dequantize(*Q.mx_quantize(np.swapaxes(v, -1, -2).astype(np.float32))), -1, -2)
    got = Q.mx_attention(q, k, v)
    np.testing.assert_allclose(got, np.broadcast_to(vq.mean(axis=2, keepdims=True), got.shape), rtol=1e-12)
    # the value quantisation runs along the keys: per key it would differ
    vk = Q.mx_dequantize(*Q.mx_quantize(v.astype(np.float32)))
    assert not np.allclose(vk.mean(axis=2), vq.mean(axis=2), rtol=1e-6)


def test_mx_attention_tracks_exact_attention():
    """Unit-scale scores: the FP8 result's RMS error against exact attention
    matches the rounding budget -- about 2.65 % RMS from the values, 2.65 %
    from the probabilities and sqrt(2) x 2.65 % on the scores (q and k),
    carried into the weights by the exponential: sqrt(2.65^2 + 2.65^2 +
    3.7^2) = 5.3 %. A dropped quantisation lowers it, a wrong axis or scale
    raises it past the band."""
    import oracle as O
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 3, 64, 128))
    k = rng.standard_normal((2, 3, 96, 128))
    v = rng.standard_normal((2, 3, 96, 128))
    ex, got = O.attention(q, k, v), Q.mx_attention(q, k, v)
    rms = np.sqrt(((got - ex) ** 2).mean() / (ex ** 2).mean())
    assert 0.03 < rms < 0.08


def test_block_routes_self_attention_through_the_hook():
    import oracle as O
    from synth import CONFIGS, make_weights, weights_f32, block_inputs
    cfg = CONFIGS["toy"]
    W = weights_f32(make_weights(cfg))
    x, e, a = block_inputs(cfg, 1)
    seen = []

    def spy(q, k, v):
        seen.append(q.shape)
        return O.attention(q, k, v)

    np.testing.assert_array_equal(O.dit_block_from_temb(x, e, a, W, 0, cfg, attn=spy),
                                  O.dit_block_from_temb(x, e, a, W, 0, cfg))
    assert seen == [(1, cfg.n_heads, cfg.tokens, cfg.head_dim)]


def test_qkv_hook_is_the_self_attention_input_projection():
    """The qkv_linear hook takes the QKV projection and nothing else: once per
    block, [B, N, D] -> [B, N, 3D] with the block's qkv weights; the default
    hook gives the plain oracle bitwise."""
    import oracle as O
    from synth import CONFIGS, make_weights, weights_f32, block_inputs
    cfg = CONFIGS["toy"]
    W = weights_f32(make_weights(cfg))
    x, e, a = block_inputs(cfg, 1)
    seen = []

    def spy(h, w, b):
        seen.append((h.shape, w.shape))
        return O.linear(h, w, b)

    np.testing.assert_array_equal(O.dit_block_from_temb(x, e, a, W, 0, cfg, qkv_linear=spy),
                                  O.dit_block_from_temb(x, e, a, W, 0, cfg))
    assert seen == [((1, cfg.tokens, cfg.dim), (3 * cfg.dim, cfg.dim))]


def _grid_ints(rng, shape):
    """Entries in {-2, -1, 0, 1, 2}: exact in e4m3 under any block scale."""
    return rng.integers(-2, 3, shape).astype(np.float64)


def test_mx_attention_identity_values_expose_the_probabilities():
    """v = identity (32 keys x 32 dims, exact under MX), q and k on the MX grid
    (so the scores are exact): the output is exactly Q(p) / sum(p), with p the
    unquantised exp(s - max) and Q the MX round trip along the keys."""
    rng = np.random.default_rng(7)
    q, k = _grid_ints(rng, (1, 1, 8, 32)), _grid_ints(rng, (1, 1, 32, 32))
    v = np.eye(32)[None, None]
    s = q @ np.swapaxes(k, -1, -2) / np.sqrt(32)
    p = np.exp(s - s.max(-1, keepdims=True))
    want = Q.mx_dequantize(*Q.mx_quantize(p.astype(np.float32))) / p.sum(-1, keepdims=True)
    np.testing.assert_allclose(Q.mx_attention(q, k, v), want, rtol=1e-13, atol=0)
    assert not np.allclose(want * p.sum(-1, keepdims=True), p, rtol=1e-6)   # the rounding is visible


@pytest.mark.parametrize("side", ["k", "q"])
def test_mx_attention_quantises_q_and_k_along_the_head_dim(side):
    """One operand one-hot (exact), the other off the grid: a score is one
    entry of the off-grid operand after its MX round trip along dh."""
    rng = np.random.default_rng(8)
    off = rng.standard_normal((1, 1, 32, 32)) * 3
    hot = np.zeros((1, 1, 32, 32))
    hot[0, 0, np.arange(32), rng.integers(0, 32, 32)] = 1.0
    q, k = (hot, off) if side == "k" else (off, hot)
    v = np.eye(32)[None, None]
    qd = Q.mx_dequantize(*Q.mx_quantize(q.astype(np.float32)))
    kd = Q.mx_dequantize(*Q.mx_quantize(k.astype(np.float32)))
    s = qd @ np.swapaxes(kd, -1, -2) / np.sqrt(32)
    p = np.exp(s - s.max(-1, keepdims=True))
    want = Q.mx_dequantize(*Q.mx_quantize(p.astype(np.float32))) / p.sum(-1, keepdims=True)
    np.testing.assert_allclose(Q.mx_attention(q, k, v), want, rtol=1e-13, atol=0)
    raw = q @ np.swapaxes(k, -1, -2) / np.sqrt(32)
    assert not np.allclose(s, raw, rtol=1e-6)                              # the round trip mattered
