"""Race check through LDS: every kernel whose waves share LDS run with its
workgroups taking their work in the reverse order (fh_debug_workgroup_order),
on a toy slice, a full-width two-block slice (every bf16 GEMM form, the
attention, norms, head), the FP8 attention and FFN path, the video decoder
and the colour match. No reduction depends on scheduling, so each output must
equal the normal order's bit for bit."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _slice_runner(fh, cfg, precision=None):
    W = synth.make_weights(cfg)
    ctx = fh.fh_create(cfg)
    w = fh.fh_weights_bind(ctx, W)
    if precision is not None:
        fh.fh_weights_quantize_fp8(ctx, w)
        fh.fh_set_option(ctx, fh.FH_OPT_PRECISION, precision)
    fh.fh_set_option(ctx, fh.FH_OPT_GRAPH, 0)      # direct launches: each run reads the flag afresh
    ws = fh.workspace(ctx, 1)
    lat, mot, aud = synth.slice_inputs(cfg, 1)
    L, Mo, A = dev(lat), dev(mot), dev(aud)

    def run():
        out = torch.empty_like(L)
        fh.fh_dit_denoise_slice(ctx, w, L, Mo, A, [1.0, 0.5, 0.0], out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    return run, (ctx, w, ws)


def _vae_runner(fh):
    vc = synth.VAE_CONFIGS["ragged"]
    vw = fh.fh_vae_weights_bind(vc, synth.make_vae_weights(vc))
    z = dev(synth.vae_latent(vc))

    def run():
        out = fh.fh_vae_decode(vw, z)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    return run, (vw,)


def _color_runner(fh):
    fr, pic = synth.color_inputs(*synth.COLOR_SHAPES["toy"])
    F, P = dev(fr), dev(pic)

    def run():
        out = fh.fh_color_match(F, P, 1.0)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    return run, (F, P)


def test_outputs_do_not_depend_on_workgroup_order(fh):
    runners = {
        "toy slice": _slice_runner(fh, synth.CONFIGS["toy"]),
        "full-width 2-block slice": _slice_runner(fh, synth.CONFIGS["slice"].replace(n_blocks=2)),
        "toy slice, FP8 FFN + attention": _slice_runner(fh, synth.CONFIGS["toy"], fh.FH_PREC_FP8_ATTN),
        "toy slice, FP8 FFN + QKV": _slice_runner(fh, synth.CONFIGS["toy"], fh.FH_PREC_FP8_QKV),
        "video decoder (ragged)": _vae_runner(fh),
        "colour match": _color_runner(fh),
    }
    normal = {k: r() for k, (r, _) in runners.items()}
    try:
        fh.fh_debug_workgroup_order(True)
        for k, (r, _) in runners.items():
            say(f"reversed workgroup order: {k}")
            np.testing.assert_array_equal(r(), normal[k], err_msg=k)
    finally:
        fh.fh_debug_workgroup_order(False)
    for k, (r, _) in runners.items():       # and back
        np.testing.assert_array_equal(r(), normal[k], err_msg=k)
