"""Throughput of the FlashHead Lite slice denoiser on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload slice|slice_b3|slice768]
                    [--sampler euler|renoise] [--precision bf16|fp8ffn|fp8qkv|fp8attn]

A step is one full slice denoise (30 blocks x 4 Euler steps, audio K/V, time
embedding, head and motion pin) of a batch of synthetic inputs already in
HBM. Prints ONE JSON line. Only one GPU is used; --gpus > 1 exits.

Extra objects on the line:
  roofline      the FFN down-projection GEMM (the longest kernel; K split in
                two halves): algorithmic FLOPs per launch / its mean duration,
                timed with HIP events on the launch stream over a second pass
                of the same K steps.
  hot_mfma_frac the method's FLOPs of every GEMM and attention kernel class
                (QKV, O, cross-q, cross-out, FFN up/down, self- and
                cross-attention, the per-slice audio K/V) / the sum of their
                kernel times / the 2.5 PF bf16 peak; per-class figures under
                "hot".
  shader_clock_mhz
                the clock every CU holds while it runs back-to-back MFMAs.
  workloads     batch 3 (three streams) and 768x768 (2880 tokens): frames/s,
                ms per call and their own hot-kernel fractions.
  fp8_options   the block-scaled FP8 precisions (FFN; FFN and QKV; FFN, QKV
                and self-attention) on the batch-1 slice: frames/s, ms per call.
  cpu_baseline  the fp32 numpy oracle on this host: one real-shape block
                (1280 tokens, its audio K/V and modulation) three times,
                median, scaled to the slice's 120 block-steps.
  audio_front_end, vae_decode, color_correction
                the audio projection before the denoise, the video decoder
                after it and the Lab colour match after the decode, each
                timed on its own.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
FRAMES_PER_SLICE = 24         # each slice emits its last 24 frames
METRIC = "DiT slice denoise video frames/s (30 blk×4 steps) + % bf16 MFMA peak"
WORKLOADS = {
    "slice": ("slice", 1, "full Lite slice denoise, batch 1: 30 blocks x 4 Euler steps, latent "
                          "16x5x16x16 (1280 tokens, 2 motion frames), 160 audio tokens, width 1536"),
    "slice_b3": ("slice", 3, "full Lite slice denoise, batch 3 (three independent streams)"),
    "slice768": ("slice768", 1, "full slice denoise at 768x768, latent 16x5x24x24 (2880 tokens), batch 1"),
}
ROOF_KERNEL = "gemm_ffn2"
COPY_BYTES = 256 << 20        # calibration copy: reads and writes this many bytes


def flops_per_slice(cfg, B, n_steps):
    """Algorithmic FLOPs of one slice call (multiply-add = 2)."""
    N, D, Fd, La = cfg.tokens, cfg.dim, cfg.ffn_dim, cfg.audio_tokens
    M = B * N
    gemm = 2 * M * D * (3 * D + D + D + D) + 2 * 2 * M * D * Fd
    attn = 4 * B * N * N * D
    keys = La if cfg.cross_full else cfg.audio_per_frame
    cross = 4 * B * N * keys * D
    per_step_blocks = cfg.n_blocks * (gemm + attn + cross)
    audio_kv = cfg.n_blocks * 2 * B * La * 2 * D * D
    time_mlp = 2 * (cfg.freq_dim * D + D * D + 6 * D * D)
    patch_head = 2 * M * cfg.in_ch * D + 2 * M * D * cfg.out_ch
    return n_steps * (per_step_blocks + time_mlp + patch_head) + audio_kv, \
        n_steps * cfg.n_blocks * (gemm + attn)


# kernel classes of the hot path (GEMMs and attention) and the method's FLOPs
# of each per slice call
HOT_CLASSES = ["gemm_qkv", "gemm_o", "gemm_cq", "gemm_co", "gemm_ffn1", "gemm_ffn2", "attn", "cross_attn",
               "audio_kv"]


def hot_flops_per_class(cfg, B, n_steps):
    """Algorithmic FLOPs per slice call of each hot kernel class. The folded
    cross-attention output executes fewer FLOPs than 2 M D D; the method's
    count is what the rate is quoted on."""
    N, D, Fd, La = cfg.tokens, cfg.dim, cfg.ffn_dim, cfg.audio_tokens
    M, bs = B * N, n_steps * cfg.n_blocks
    keys = La if cfg.cross_full else cfg.audio_per_frame
    return {"gemm_qkv": bs * 2 * M * D * 3 * D, "gemm_o": bs * 2 * M * D * D, "gemm_cq": bs * 2 * M * D * D,
            "gemm_co": bs * 2 * M * D * D, "gemm_ffn1": bs * 2 * M * D * Fd, "gemm_ffn2": bs * 2 * M * Fd * D,
            "attn": bs * 4 * B * N * N * D, "cross_attn": bs * 4 * M * keys * D,
            "audio_kv": cfg.n_blocks * 2 * B * La * D * 2 * D}


def hot_fraction(per_class_ms, flops):
    """(hot TF/s, fraction of the bf16 peak) from per-slice ms and FLOPs of the classes."""
    t = sum(per_class_ms[k] for k in flops) * 1e-3
    f = sum(flops.values())
    return f / t / 1e12, f / t / 1e12 / PEAK_BF16_TFLOPS


def time_classes(fh, ctx, step, torch, classes, passes):
    """ms per slice call and launches per call of each kernel class: HIP events
    around its launches over `passes` calls (direct launches)."""
    out = {}
    for name in classes:
        fh.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, fh.FH_K[name])
        step()
        torch.cuda.synchronize()
        fh.fh_kernel_time(ctx)
        for _ in range(passes):
            step()
        torch.cuda.synchronize()
        ms, n = fh.fh_kernel_time(ctx)
        out[name] = (ms / passes, n / passes)
    fh.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, -1)
    return out


def hot_report(timed, flops):
    per = {}
    for k, f in flops.items():
        ms, n = timed[k]
        tf = f / (ms * 1e-3) / 1e12
        per[k] = {"ms_per_call": round(ms, 4), "launches_per_call": round(n, 2), "gflop_per_call": round(f / 1e9, 2),
                  "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    tf, frac = hot_fraction({k: v[0] for k, v in timed.items()}, flops)
    return per, round(tf, 1), round(frac, 4), round(sum(timed[k][0] for k in flops), 4)


def blas_threads():
    import threadpoolctl
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    return int(max([p.get("num_threads", 1) for p in blas] or [1]))


def oracle_beside(name, gpu_us):
    """The float64 oracle of a secondary row (audio front end, video decoder,
    colour match) timed once at the bench's own size on the host, beside the
    GPU's time: a reported baseline, not a target."""
    import synth
    if name == "audio_front_end":
        from oracle import audio as AU
        acfg = synth.AUDIO_CONFIGS["lite"]
        S, Wa = synth.audio_states(acfg, 1), synth.weights_f32(synth.make_audio_weights(acfg))
        t0 = time.perf_counter()
        AU.audio_project(S, Wa, acfg)
        sample = "one batch-1 projection, float64 numpy"
    elif name == "vae_decode":
        from oracle import vae as V
        vc = synth.VAE_CONFIGS["slice"]
        W = synth.vae_weights_f32(synth.make_vae_weights(vc))
        z = synth.vae_latent(vc)
        t0 = time.perf_counter()
        V.decode(z, W, vc)
        sample = "one slice decode (33 x 512 x 512), float64 numpy with the F16 storage points"
    else:
        from oracle import color as C
        F, H, W, Hr, Wr = synth.COLOR_SHAPES["slice"]
        fr, pic = synth.color_inputs(F, H, W, Hr, Wr)
        t0 = time.perf_counter()
        C.color_match(fr, pic, 1.0)
        sample = "one slice colour match (33 frames of 512 x 512), float64 numpy"
    t = time.perf_counter() - t0
    return {"s_per_call": round(t, 3), "kind": "oracle", "cores": blas_threads(), "sample": sample,
            "gpu_speedup": round(t / (gpu_us * 1e-6), 1)}


def cpu_baseline(cfg, sigmas, repeats=3):
    """The fp32 numpy oracle on one real-shape block (1280 tokens: modulation
    from a time embedding, the block's audio K/V, the block), `repeats` times;
    the median, times the slice's block-steps, gives the slice time."""
    import threadpoolctl
    import oracle
    import synth
    W = synth.weights_f32(synth.make_weights(cfg, blocks=[0]))
    x, e, a = synth.block_inputs(cfg, 1)
    ts = []
    with oracle.working_dtype(np.float32):
        for _ in range(repeats):
            t0 = time.perf_counter()
            oracle.dit_block_from_temb(x, e, a, W, 0, cfg)
            ts.append(time.perf_counter() - t0)
    t_block = sorted(ts)[len(ts) // 2]
    block_steps = cfg.n_blocks * (len(sigmas) - 1)
    t_slice = t_block * block_steps
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    cpu = "unknown"
    try:
        cpu = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    flops = sum(hot_flops_per_class(cfg, 1, len(sigmas) - 1).values()) / block_steps
    return {"value": FRAMES_PER_SLICE / t_slice, "unit": "frames/s", "cores": int(threads),
            "kind": "oracle", "cpu": cpu,
            "blas": ", ".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip() for p in blas})),
            "block_s_median": round(t_block, 4), "block_s_all": [round(t, 4) for t in ts],
            "gflops": round(flops / t_block / 1e9, 1),
            "sample": f"one real-shape block (1280 tokens, width {cfg.dim}, its audio K/V and modulation) run "
                      f"{repeats} times by the float32 numpy oracle, median {t_block:.3f} s, times the "
                      f"{block_steps} block-steps of a batch-1 slice"}


def audio_front_end(fh, torch, ctx, cfg, B, stream, calls):
    """Time the audio projection (speech-encoder states -> the slice's audio
    tokens, once per slice) on its own: HIP events around `calls` calls. It
    streams its bf16 weights once per call, so its bound is HBM."""
    import synth
    acfg = synth.AUDIO_CONFIGS["lite"]
    Wa = synth.make_audio_weights(acfg)
    wbytes = sum(a.nbytes for a in Wa.values())
    aw = fh.fh_audio_weights_bind(ctx, acfg, Wa)
    del Wa
    ws = fh.audio_workspace(aw, B)
    S = torch.from_numpy(synth.audio_states(acfg, B)).cuda()
    tok = torch.empty(B, cfg.audio_tokens, cfg.dim, dtype=torch.float32, device="cuda")
    for _ in range(3):
        fh.fh_audio_project(ctx, aw, S, tok, ws, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        fh.fh_audio_project(ctx, aw, S, tok, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    # algorithmic bytes: the weights once, the states once, the tokens written
    alg = wbytes + S.numel() * 4 + tok.numel() * 4
    return {"us_per_call": round(us, 2), "calls_timed": calls, "bound": "hbm",
            "algorithmic_bytes": int(alg), "achieved_GBps": round(alg / (us * 1e-6) / 1e9, 1),
            "peak_GBps": PEAK_HBM_GBS, "frac": round(alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "workload": f"audio projection, batch {B}: 12 x 200 x 768 states -> {cfg.audio_tokens} tokens of "
                        f"width {cfg.dim} (proj1/proj1vf 46080 -> 512, proj2, proj3 512 -> 32 x 1536, "
                        f"LayerNorm)"}


def color_correction(fh, torch, stream, calls):
    """Time the Lab colour match of one slice's decoded frames (33 of 512 x 512,
    RGB planes) to the 512 x 512 picture, strength 1: HIP events around
    `calls` calls on the launch stream. Algorithmic bytes: the frames read
    once and written once, the picture read once (the statistics must see
    every pixel before any output, so the kernels read the frames twice)."""
    import synth
    F, H, W, Hr, Wr = synth.COLOR_SHAPES["slice"]
    fr, pic = synth.color_inputs(F, H, W, Hr, Wr)
    Fd, Pd = torch.from_numpy(fr).cuda(), torch.from_numpy(pic).cuda()
    out = torch.empty_like(Fd)
    ws = torch.empty(fh.fh_color_match_workspace_bytes(F, H, W, Hr, Wr), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        fh.fh_color_match(Fd, Pd, 1.0, out=out, workspace=ws, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        fh.fh_color_match(Fd, Pd, 1.0, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    alg = 4 * (2 * fr.size + pic.size)
    gbs = alg / (us * 1e-6) / 1e9
    return {"us_per_call": round(us, 2), "calls_timed": calls, "bound": "hbm", "algorithmic_bytes": int(alg),
            "achieved_GBps": round(gbs, 1), "peak_GBps": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
            "frames_per_s": round(F * calls / (e0.elapsed_time(e1) * 1e-3), 1),
            "workload": f"Lab colour match, strength 1: {F} decoded frames of {H}x{W} (float32 RGB planes) "
                        f"to the {Hr}x{Wr} picture"}


def other_workload(fh, torch, synth, W, name, stream, steps, hot_passes, no_graph):
    """frames/s, ms per call and the hot-kernel fraction of another workload of
    the metric's configuration list (batch 3, 768x768), on the same weights."""
    cfg_name, B, desc = WORKLOADS[name]
    cfg = synth.CONFIGS[cfg_name]
    sig = list(synth.SLICE_SIGMAS)
    ctx = fh.fh_create(cfg)
    w = fh.fh_weights_bind(ctx, W)
    ws = fh.workspace(ctx, B)
    L, Mo, A = (torch.from_numpy(a).cuda() for a in synth.slice_inputs(cfg, B))
    out = torch.empty_like(L)
    fh.fh_set_option(ctx, fh.FH_OPT_GRAPH, 0 if no_graph else 1)

    def step():
        fh.fh_dit_denoise_slice(ctx, w, L, Mo, A, sig, out, ws, stream)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    T = time.perf_counter() - t0
    total, _ = flops_per_slice(cfg, B, len(sig) - 1)
    timed = time_classes(fh, ctx, step, torch, HOT_CLASSES, hot_passes)
    per, tf, frac, ms_hot = hot_report(timed, hot_flops_per_class(cfg, B, len(sig) - 1))
    res = {"workload": desc, "batch": B, "tokens": cfg.tokens, "steps": steps,
           "frames_per_s": round(FRAMES_PER_SLICE * B * steps / T, 2), "ms_per_call": round(1e3 * T / steps, 4),
           "tflops_end_to_end": round(total / (T / steps) / 1e12, 2), "hot_mfma_frac": frac, "hot_tflops": tf,
           "hot_ms_per_call": ms_hot, "attn": per["attn"], "gemm_ffn2": per["gemm_ffn2"]}
    del w, ws, L, Mo, A, out
    torch.cuda.empty_cache()
    return res


def fp8_options(fh, torch, synth, W, stream, steps, no_graph):
    """frames/s and ms per call of the block-scaled FP8 precisions on the batch-1
    slice and the same weights (quantised once): FFN; FFN and QKV; FFN, QKV and
    self-attention. Options, not the metric's configuration."""
    cfg = synth.CONFIGS["slice"]
    sig = list(synth.SLICE_SIGMAS)
    ctx = fh.fh_create(cfg)
    w = fh.fh_weights_bind(ctx, W)
    fh.fh_weights_quantize_fp8(ctx, w)
    fh.fh_set_option(ctx, fh.FH_OPT_GRAPH, 0 if no_graph else 1)
    L, Mo, A = (torch.from_numpy(a).cuda() for a in synth.slice_inputs(cfg, 1))
    out = torch.empty_like(L)
    total, _ = flops_per_slice(cfg, 1, len(sig) - 1)
    res = {}
    for name, prec in (("fp8ffn", fh.FH_PREC_FP8_FFN), ("fp8qkv", fh.FH_PREC_FP8_QKV),
                       ("fp8attn", fh.FH_PREC_FP8_ATTN)):
        fh.fh_set_option(ctx, fh.FH_OPT_PRECISION, prec)
        ws = fh.workspace(ctx, 1)  # sized for the precision

        def step():
            fh.fh_dit_denoise_slice(ctx, w, L, Mo, A, sig, out, ws, stream)

        for _ in range(2):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        T = time.perf_counter() - t0
        res[name] = {"frames_per_s": round(FRAMES_PER_SLICE * steps / T, 2), "ms_per_call": round(1e3 * T / steps, 4),
                     "tflops_end_to_end": round(total / (T / steps) / 1e12, 2), "steps": steps}
        del ws
    del w, L, Mo, A, out
    torch.cuda.empty_cache()
    return res


def vae_flops(vc):
    """Algorithmic FLOPs of one decode: 2 x 27 C_in C_out per output position of
    every convolution (the norms, SiLU and depth to space are bytes, not FLOPs)."""
    T, H, W, w = vc.frames, vc.height, vc.width, vc.widths
    f = 2 * 27 * vc.latent_ch * w[0] * T * H * W
    for i in range(3):
        f += 2 * (2 * 27 * w[i] * w[i] * T * H * W) + 2 * 27 * w[i] * 8 * w[i + 1] * T * H * W
        T, H, W = 2 * T - 1, 2 * H, 2 * W
    return f + 2 * 27 * w[3] * vc.out_ch * vc.patch ** 2 * T * H * W


def vae_decode(fh, torch, synth, stream, calls):
    """Time the video decoder on one slice latent (5 x 16 x 16 -> 33 frames of
    512 x 512): HIP events around `calls` calls on the launch stream; its
    convolutions are F16 MFMA contractions, priced against the 2.5 PF dense
    F16/bf16 peak."""
    vc = synth.VAE_CONFIGS["slice"]
    vw = fh.fh_vae_weights_bind(vc, synth.make_vae_weights(vc))
    z = torch.from_numpy(synth.vae_latent(vc)).cuda()
    out = torch.empty(3, vc.out_frames, vc.out_height, vc.out_width, device="cuda")
    ws = torch.empty(fh.fh_vae_workspace_bytes(vc), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        fh.fh_vae_decode(vw, z, out, ws, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        fh.fh_vae_decode(vw, z, out, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    fl = vae_flops(vc)
    tf = fl / (us * 1e-6) / 1e12
    return {"us_per_call": round(us, 1), "calls_timed": calls, "bound": "mfma", "gflop_per_call": round(fl / 1e9, 2),
            "tflops": round(tf, 1), "peak_tflops": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "frames_per_s": round(vc.out_frames * calls / (e0.elapsed_time(e1) * 1e-3), 1),
            "workload": f"video decoder, one slice latent {vc.latent_ch}x{vc.frames}x{vc.height}x{vc.width} -> "
                        f"{vc.out_frames} frames of {vc.out_height}x{vc.out_width}, widths {list(vc.widths)}, "
                        "F16 operands, F32 sums"}


def device_info(torch):
    """Name, compute units and L2 size of cuda:0 as the runtime reports them."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "compute_units": p.multi_processor_count,
            "gcn_arch": getattr(p, "gcnArchName", ""), "l2_bytes": getattr(p, "L2_cache_size", None)}


def kernel_code_hash(path):
    """SHA-256 of a kernel source's code: // comments, trailing blanks and empty
    lines removed, so an edit of comments alone keeps counters taken on the
    same code valid."""
    lines = []
    for line in open(path, encoding="utf-8"):
        code = re.sub(r"//.*$", "", line).rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def traffic_from_profile(kernel_src_hash, name):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3
    counter summary profiles/<name> (FETCH_SIZE and WRITE_SIZE scaled by a copy
    kernel of known size), if it was taken on the current kernel code
    (kernel_code_hash); else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("code_sha256") != kernel_src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="slice", choices=sorted(WORKLOADS))
    ap.add_argument("--sampler", default="euler", choices=["euler", "renoise"],
                    help="step update: Euler (the metric's configuration) or the re-noising variant")
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp8ffn", "fp8qkv", "fp8attn"],
                    help="bf16 everywhere (the metric's configuration); fp8ffn: the FFN's two GEMMs in "
                         "block-scaled FP8 (MX e4m3, one power-of-two scale per 32 along K); fp8qkv: "
                         "those and the QKV projection; fp8attn: those and the self-attention")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="time every kernel class (slow)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the batch-3 and 768x768 workloads and the per-class hot-kernel timing")
    ap.add_argument("--hot-passes", type=int, default=3, help="slice calls per timed kernel class")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one elementwise copy of 256 MiB (read + write) first; rocprofv3 "
                         "counter runs use it to scale FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the slice denoiser is a "
              "single-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import audio_driven_talking_amd as fh
    import synth

    cfg_name, B, desc = WORKLOADS[args.workload]
    cfg = synth.CONFIGS[cfg_name]
    sig = list(synth.SLICE_SIGMAS)
    n_steps = len(sig) - 1
    W = synth.make_weights(cfg)
    ctx = fh.fh_create(cfg)
    w = fh.fh_weights_bind(ctx, W)
    fp8 = args.precision in ("fp8ffn", "fp8qkv", "fp8attn")
    if fp8:
        fh.fh_weights_quantize_fp8(ctx, w)
        fh.fh_set_option(ctx, fh.FH_OPT_PRECISION,
                         {"fp8ffn": fh.FH_PREC_FP8_FFN, "fp8qkv": fh.FH_PREC_FP8_QKV,
                          "fp8attn": fh.FH_PREC_FP8_ATTN}[args.precision])
    ws = fh.workspace(ctx, B)
    lat, mot, aud = synth.slice_inputs(cfg, B)
    L, Mo, A = (torch.from_numpy(a).cuda() for a in (lat, mot, aud))
    out = torch.empty_like(L)
    fh.fh_set_option(ctx, fh.FH_OPT_GRAPH, 0 if args.no_graph else 1)
    if args.sampler == "renoise":
        fh.fh_set_option(ctx, fh.FH_OPT_SAMPLER, fh.FH_SAMPLER_RENOISE)
        fh.fh_set_noise_seed(ctx, 20240601)
    stream = torch.cuda.current_stream()
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step():
        fh.fh_dit_denoise_slice(ctx, w, L, Mo, A, sig, out, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    T = time.perf_counter() - t0
    ms = 1e3 * T / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    p50 = per_step[len(per_step) // 2]
    p90 = per_step[min(len(per_step) - 1, int(0.9 * len(per_step)))]

    total_flops, hot_flops = flops_per_slice(cfg, B, n_steps)
    value = FRAMES_PER_SLICE * B * args.steps / T

    # roofline kernel: HIP events around each FFN-down launch, same K steps, direct launches
    fh.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, fh.FH_K[ROOF_KERNEL])
    step()
    torch.cuda.synchronize()
    fh.fh_kernel_time(ctx)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kms, kn = fh.fh_kernel_time(ctx)
    fh.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, -1)
    M = B * cfg.tokens
    k_flops = 2.0 * M * cfg.ffn_dim * cfg.dim
    k_avg_s = kms / 1e3 / max(kn, 1)
    achieved = k_flops / k_avg_s / 1e12
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    code_hash = kernel_code_hash(os.path.join(ROOT, "audio_driven_talking_amd", "csrc", "gemm.hip"))
    counters = "gemm_mx_ffn2_slice_b1_counters.json" if fp8 else "gemm_ffn2_slice_b1_counters.json"
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic_from_profile(code_hash, counters),
                "kernel": f"{ROOF_KERNEL} (M={M}, N={cfg.dim}, K={cfg.ffn_dim}, "
                          f"{'MX-FP8 e4m3' if fp8 else 'bf16'}, {k_flops / 1e9:.2f} GFLOP per launch)",
                "avg_us": round(k_avg_s * 1e6, 2), "launches_timed": kn}

    # every GEMM and attention class: the hot-path fraction of the MFMA peak
    hot = None
    if not args.no_extra and not fp8:
        timed = time_classes(fh, ctx, step, torch, [k for k in HOT_CLASSES if k != ROOF_KERNEL], args.hot_passes)
        timed[ROOF_KERNEL] = (kms / max(args.steps, 1), kn / max(args.steps, 1))
        hot = hot_report(timed, hot_flops_per_class(cfg, B, n_steps))
    clock = fh.fh_shader_clock(stream=stream)

    # the other workloads of the metric's configuration list, same weights
    extra = {}
    fp8_opts = None
    if not args.no_extra and args.workload == "slice" and not fp8 and args.sampler == "euler":
        for name in ("slice_b3", "slice768"):
            extra[name] = other_workload(fh, torch, synth, W, name, stream, max(3, args.steps // 2),
                                         args.hot_passes, args.no_graph)
        fp8_opts = fp8_options(fh, torch, synth, W, stream, args.steps, args.no_graph)
    del W

    front = audio_front_end(fh, torch, ctx, cfg, B, stream, args.steps) if cfg_name == "slice" else None
    color = color_correction(fh, torch, stream, args.steps) if cfg_name == "slice" else None
    vae = vae_decode(fh, torch, synth, stream, max(5, args.steps // 2)) if cfg_name == "slice" else None

    breakdown = None
    if args.breakdown:
        breakdown = {}
        for name, k in fh.FH_K.items():
            fh.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, k)
            fh.fh_kernel_time(ctx)
            for _ in range(3):
                step()
            torch.cuda.synchronize()
            t, n = fh.fh_kernel_time(ctx)
            breakdown[name] = {"ms_per_slice": round(t / 3, 4), "launches_per_slice": n // 3}
        fh.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, -1)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8ffn": "bf16, FFN GEMMs mxfp8 (e4m3)",
                  "fp8qkv": "bf16, FFN and QKV GEMMs mxfp8 (e4m3)",
                  "fp8attn": "bf16, FFN GEMMs and self-attention mxfp8 (e4m3)"}[args.precision],
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) latent/motion/audio)",
        "config": {"workload": desc, "batch": B, "tokens": cfg.tokens, "blocks": cfg.n_blocks,
                   "euler_steps": n_steps, "dim": cfg.dim, "heads": cfg.n_heads,
                   "ffn": cfg.ffn_dim, "audio_tokens": cfg.audio_tokens,
                   "cross_attention": "full" if cfg.cross_full else "frame-local",
                   "sampler": args.sampler, "precision": args.precision,
                   "graph": not args.no_graph},
        "ms_per_step_p50": round(p50, 4), "ms_per_step_p90": round(p90, 4),
        "latent_token_steps_per_s": round(B * cfg.tokens * n_steps * args.steps / T, 1),
        "device": device_info(torch),
        "mfma_frac_end_to_end": round(total_flops / (T / args.steps) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "tflops_end_to_end": round(total_flops / (T / args.steps) / 1e12, 2),
        "roofline": roofline,
        "shader_clock_mhz": round(clock, 1),
    }
    if hot is not None:
        per, tf, frac, ms_hot = hot
        line["hot_mfma_frac"] = frac
        line["hot_tflops"] = tf
        line["hot"] = {"classes": per, "ms_per_call": ms_hot, "ms_per_call_all_kernels_wall": round(ms, 4),
                       "peak_tflops": PEAK_BF16_TFLOPS,
                       "peak_at_measured_clock_tflops": round(PEAK_BF16_TFLOPS * clock / 2400.0, 1)}
    if extra:
        line["workloads"] = extra
    if fp8_opts is not None:
        line["fp8_options"] = fp8_opts
    if front is not None:
        line["audio_front_end"] = front
    if vae is not None:
        line["vae_decode"] = vae
    if color is not None:
        line["color_correction"] = color
    if breakdown is not None:
        line["kernel_ms_per_slice"] = breakdown
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, sig)
        for k in ("audio_front_end", "vae_decode", "color_correction"):
            if k in line:
                line[k]["cpu_oracle"] = oracle_beside(k, line[k]["us_per_call"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
