"""Write the expected outputs of the full-size slice parity tests.

Calls only the CPU oracle (float64) on the seeded synthetic data:
    python tests/golden/make_golden.py [slice_b1 slice_b3 slice768 slice_b1_renoise slice_b1_fp8ffn]
Each case is saved as <case>.npz with the output latent (float32), the
weights digest, the sigma schedule, the sampler and the FFN product (exact
float64, or the MX-FP8 product of both operands), so a test can check it is comparing
against the same weights.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

CASES = {  # name: (configuration, batch, sampler, FFN product)
    "slice_b1": ("slice", 1, "euler", "exact"),
    "slice_b3": ("slice", 3, "euler", "exact"),
    "slice768": ("slice768", 1, "euler", "exact"),
    "slice_b1_renoise": ("slice", 1, "renoise", "exact"),
    "slice_b1_fp8ffn": ("slice", 1, "euler", "mxfp8"),
}
NOISE_SEED = 20240601  # seed of the re-noising sampler's noise


def make(case):
    cfg_name, batch, sampler, ffn = CASES[case]
    ffn_linear = oracle.mxfp8.mx_linear if ffn == "mxfp8" else oracle.linear
    cfg = synth.CONFIGS[cfg_name]
    W = synth.make_weights(cfg)
    Wf = synth.weights_f32(W)
    lat, mot, aud = synth.slice_inputs(cfg, batch)
    sig = list(synth.SLICE_SIGMAS)
    t = time.time()
    if sampler == "euler":
        # lanes are independent: one lane at a time keeps the memory small
        out = np.concatenate([oracle.denoise_slice(lat[b:b + 1], mot[b:b + 1], aud[b:b + 1], sig, Wf, cfg,
                                                    ffn_linear=ffn_linear)
                              for b in range(batch)])
    else:  # the noise counter carries the lane index: the whole batch at once
        assert ffn == "exact"
        out = oracle.renoise.denoise_slice_renoise(lat, mot, aud, sig, Wf, cfg, NOISE_SEED)
    np.savez(os.path.join(HERE, case + ".npz"), out=out.astype(np.float32),
             digest=np.array(synth.weights_digest(W)), sigmas=np.array(sig), config=np.array(cfg_name),
             batch=np.array(batch), sampler=np.array(sampler), ffn=np.array(ffn), noise_seed=np.array(NOISE_SEED))
    print(f"{case}: {time.time() - t:.1f}s", flush=True)


if __name__ == "__main__":
    for c in (sys.argv[1:] or list(CASES)):
        make(c)
