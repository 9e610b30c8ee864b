"""The allocation-free colour match, fh_color_match_noalloc, called through
the C ABI (ctypes on libfh), against the workspace entry point
fh_color_match on the same inputs: the same kernels, so the outputs must be
equal bit for bit. Two calls in a row, the second on a smaller input, check
that the shared static scratch keeps no state a call depends on; a call whose
statistics exceed the scratch is rejected on the host before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def say(msg):
    print(msg, flush=True)


def noalloc(fh, F, P, strength, out):
    _, n, H, W = F.shape
    _, Hr, Wr = P.shape
    st = fh.lib.fh_color_match_noalloc(ctypes.c_void_p(F.data_ptr()), n, H, W, ctypes.c_void_p(P.data_ptr()), Hr, Wr,
                                       ctypes.c_float(strength), ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_equals_the_workspace_entry_point(fh):
    assert fh.lib.fh_color_match_noalloc_max_bytes() == 4 << 20
    for shape, strength in (("slice", 1.0), ("toy", 0.7), ("ragged", 1.0)):
        say(f"noalloc colour match, {shape} {synth.COLOR_SHAPES[shape]}, strength {strength}")
        fr, pic = synth.color_inputs(*synth.COLOR_SHAPES[shape])
        F, P = dev(fr), dev(pic)
        want = fh.fh_color_match(F, P, strength)
        out = torch.full_like(F, float("nan"))
        assert noalloc(fh, F, P, strength, out) == fh.FH_OK
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"{shape}: differs from fh_color_match"
    # in place, and again on the same buffers
    fr, pic = synth.color_inputs(*synth.COLOR_SHAPES["toy"])
    want = fh.fh_color_match(dev(fr), dev(pic), 1.0)
    F = dev(fr)
    assert noalloc(fh, F, dev(pic), 1.0, F) == fh.FH_OK
    torch.cuda.synchronize()
    assert torch.equal(F, want)


def test_noalloc_rejects_sizes_beyond_its_scratch(fh):
    """33 frames of 3840 x 2160 need 6.6 MB of statistics: FH_EWORKSPACE, found
    on the host (the pointers are never dereferenced)."""
    need = fh.fh_color_match_workspace_bytes(33, 2160, 3840, 512, 512)
    assert need > fh.lib.fh_color_match_noalloc_max_bytes()
    a, b = ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 41)
    st = fh.lib.fh_color_match_noalloc(a, 33, 2160, 3840, a, 512, 512, ctypes.c_float(1.0), b, None)
    assert st == fh.FH_EWORKSPACE
    assert fh.fh_color_match_workspace_bytes(33, 1080, 1920, 512, 512) <= fh.lib.fh_color_match_noalloc_max_bytes()
