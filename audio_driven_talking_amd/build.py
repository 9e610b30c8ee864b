"""Build libfh.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python audio_driven_talking_amd/build.py   (or __graft_entry__.build())
    FH_DEBUG=1 python audio_driven_talking_amd/build.py   -> libfh_debug.so

Every source is compiled on each call; the shared library lands next to this
file, where the binding loads it from. The debug library (the same kernels;
the runtime synchronises after every launch and captures no graphs) is what
the binding loads when FH_DEBUG=1 is set in the environment.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfh.so")
SOURCES = ["gemm.hip", "norm.hip", "attn.hip", "misc.hip", "debug_f32.hip", "audio.hip", "color.hip", "vae.hip",
           "fh_api.cpp"]
# attention keeps its MFMA accumulators in VGPRs: the online softmax rescales
# and reads them with VALU every key block, and AGPR copies would dominate.
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(OBJ + ("_debug" if debug else ""), os.path.splitext(src)[0] + ".o")
    dbg = ["-DFH_DEBUG"] if debug and src == "fh_api.cpp" else []
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *dbg, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug: bool | None = None) -> str:
    if debug is None:
        debug = os.environ.get("FH_DEBUG") == "1"
    lib = os.path.join(HERE, "libfh_debug.so") if debug else LIB
    os.makedirs(OBJ + ("_debug" if debug else ""), exist_ok=True)
    with cf.ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
