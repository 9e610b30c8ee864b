"""Write the expected outputs of the full-size slice parity tests.

Calls only the CPU oracle (float64) on the seeded synthetic data:
    python tests/golden/make_golden.py [slice_b1 slice_b3 slice768 slice_b1_renoise]
Each case is saved as <case>.npz with the output latent (float32), the
weights digest and the sigma schedule, so a test can check it is comparing
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

CASES = {  # name: (configuration, batch, sampler)
    "slice_b1": ("slice", 1, "euler"),
    "slice_b3": ("slice", 3, "euler"),
    "slice768": ("slice768", 1, "euler"),
    "slice_b1_renoise": ("slice", 1, "renoise"),
}
NOISE_SEED = 20240601  # seed of the re-noising sampler's noise


def make(case):
    cfg_name, batch, sampler = CASES[case]
    cfg = synth.CONFIGS[cfg_name]
    W = synth.make_weights(cfg)
    Wf = synth.weights_f32(W)
    lat, mot, aud = synth.slice_inputs(cfg, batch)
    sig = list(synth.SLICE_SIGMAS)
    t = time.time()
    if sampler == "euler":
        # lanes are independent: one lane at a time keeps the memory small
        out = np.concatenate([oracle.denoise_slice(lat[b:b + 1], mot[b:b + 1], aud[b:b + 1], sig, Wf, cfg)
                              for b in range(batch)])
    else:  # the noise counter carries the lane index: the whole batch at once
        out = oracle.renoise.denoise_slice_renoise(lat, mot, aud, sig, Wf, cfg, NOISE_SEED)
    np.savez(os.path.join(HERE, case + ".npz"), out=out.astype(np.float32),
             digest=np.array(synth.weights_digest(W)), sigmas=np.array(sig), config=np.array(cfg_name),
             batch=np.array(batch), sampler=np.array(sampler), noise_seed=np.array(NOISE_SEED))
    print(f"{case}: {time.time() - t:.1f}s", flush=True)


if __name__ == "__main__":
    for c in (sys.argv[1:] or list(CASES)):
        make(c)
