"""The launch trace: FH_TRACE=1 makes every kernel launch print its kernel,
grid, block, LDS bytes, stream and scalar arguments on stderr.

The environment variable is read once per process, so each case runs a toy
slice (captured as a graph, which is when its launches are issued) and a toy
block (direct launches) in a child process.
"""
import os
import re
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
import audio_driven_talking_amd as fh
import synth
cfg = synth.CONFIGS["toy"]
W = synth.make_weights(cfg)
ctx = fh.fh_create(cfg)
w = fh.fh_weights_bind(ctx, W)
ws = fh.workspace(ctx, 1)
lat, mot, aud = (torch.from_numpy(a).cuda() for a in synth.slice_inputs(cfg, 1))
out = torch.empty_like(lat)
fh.fh_dit_denoise_slice(ctx, w, lat, mot, aud, list(synth.TOY_SIGMAS), out, ws)
torch.cuda.synchronize()
print("slice done", flush=True)
"""

LINE = re.compile(r"^fh launch (\S.*?) grid (\d+)x(\d+)x(\d+) block (\d+)x(\d+)x(\d+) lds (\d+) stream (\S+) \((.*)\)$")


def run_child(trace):
    env = dict(os.environ)
    env.pop("FH_TRACE", None)
    if trace:
        env["FH_TRACE"] = "1"
    print(f"child process, FH_TRACE={'1' if trace else 'unset'}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "slice done" in r.stdout
    return [ln for ln in r.stderr.splitlines() if ln.startswith("fh launch ")]


def test_trace_lines_name_every_kernel_with_grid_and_shape():
    lines = run_child(True)
    assert lines, "no launch was traced"
    kernels = set()
    for ln in lines:
        m = LINE.match(ln)
        assert m, ln
        name = m.group(1)
        grid = tuple(int(m.group(i)) for i in (2, 3, 4))
        block = tuple(int(m.group(i)) for i in (5, 6, 7))
        assert min(grid) >= 1 and min(block) >= 1 and block[0] * block[1] * block[2] <= 1024, ln
        kernels.add(name.split("<")[0])
        if name == "layernorm_kernel":
            # arguments (x, out, rows, D, ...): one workgroup per row
            args = [a.strip() for a in m.group(10).split(",")]
            assert grid[0] == int(args[2]), ln
    for k in ("patch_embed_kernel", "layernorm_kernel", "gemm_bf16_nt", "rmsnorm_rope_kernel", "flash_attn_kernel",
              "head_euler_kernel"):
        assert k in kernels, (k, sorted(kernels))


def test_no_trace_without_the_variable():
    assert run_child(False) == []
