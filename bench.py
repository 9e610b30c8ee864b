"""Throughput of the FlashHead Lite slice denoiser on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload slice|slice_b3|slice768]
                    [--sampler euler|renoise] [--precision bf16|fp8ffn]

A step is one full slice denoise (30 blocks x 4 Euler steps, audio K/V, time
embedding, head and motion pin) of a batch of synthetic inputs already in
HBM. Prints ONE JSON line. Only one GPU is used; --gpus > 1 exits.

Extra objects on the line:
  roofline      the FFN down-projection GEMM (the longest kernel; K split in
                two halves): algorithmic FLOPs per launch / its mean duration,
                timed with HIP events on the launch stream over a second pass
                of the same K steps.
  cpu_baseline  the float64 numpy oracle timed on this host on a bounded
                sample of the same workload (some of the slice's block-steps),
                scaled to frames/s.
  audio_front_end, color_correction
                the audio projection before the denoise and the Lab colour
                match after the decode, each timed on its own.
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


def cpu_baseline(cfg, sigmas, budget_s=15.0):
    """Time the float64 oracle on block-steps of the first step, scale to a slice."""
    import threadpoolctl
    import oracle
    import synth
    W = synth.weights_f32(synth.make_weights(cfg, blocks=list(range(min(cfg.n_blocks, 8)))))
    lat, mot, aud = synth.slice_inputs(cfg, 1)
    x0 = oracle.pin_motion(lat, mot)
    e, e0 = oracle.time_embedding(np.array([sigmas[0]]), W, cfg)
    ang = oracle.rope_angles(cfg)
    x = oracle.linear(oracle.patchify(x0), W["patch.w"], W["patch.b"])
    t0 = time.perf_counter()
    k = 0
    while k < min(cfg.n_blocks, 8):
        x = oracle.dit_block(x, e0, aud, oracle.block_weights(W, k), cfg, ang)
        k += 1
        if time.perf_counter() - t0 > budget_s:
            break
    t_block = (time.perf_counter() - t0) / k
    t_slice = t_block * cfg.n_blocks * (len(sigmas) - 1)
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    cpu = "unknown"
    try:
        cpu = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": FRAMES_PER_SLICE / t_slice, "unit": "frames/s", "cores": int(threads),
            "kind": "oracle", "cpu": cpu,
            "blas": ", ".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip() for p in blas})),
            "sample": f"{k} of the {cfg.n_blocks * (len(sigmas) - 1)} block-steps of one batch-1 "
                      f"slice (float64 numpy oracle, {t_block:.3f} s per block-step), scaled to the "
                      f"whole slice"}


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
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp8ffn", "fp8attn"],
                    help="bf16 everywhere (the metric's configuration); fp8ffn: the FFN's two GEMMs in "
                         "block-scaled FP8 (MX e4m3, one power-of-two scale per 32 along K); fp8attn: "
                         "those and the self-attention")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="time every kernel class (slow)")
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
    del W
    fp8 = args.precision in ("fp8ffn", "fp8attn")
    if fp8:
        fh.fh_weights_quantize_fp8(ctx, w)
        fh.fh_set_option(ctx, fh.FH_OPT_PRECISION,
                         fh.FH_PREC_FP8_ATTN if args.precision == "fp8attn" else fh.FH_PREC_FP8_FFN)
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

    front = audio_front_end(fh, torch, ctx, cfg, B, stream, args.steps) if cfg_name == "slice" else None
    color = color_correction(fh, torch, stream, args.steps) if cfg_name == "slice" else None

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
    }
    if front is not None:
        line["audio_front_end"] = front
    if color is not None:
        line["color_correction"] = color
    if breakdown is not None:
        line["kernel_ms_per_slice"] = breakdown
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, sig)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
