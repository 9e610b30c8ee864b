"""The C ABI on the host: exports, configuration checks, weight index checks and
argument validation. Nothing here launches a kernel, so no GPU is needed."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

fh = pytest.importorskip("audio_driven_talking_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    txt = open(os.path.join(ROOT, "include", "fh.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fh_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 13
    assert sorted(fh.EXPORTS) == names
    lib = ctypes.CDLL(fh.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def cfg_dict(name="slice", **kw):
    c = synth.CONFIGS[name]
    d = {f: getattr(c, f) for f in ("n_blocks", "dim", "n_heads", "head_dim", "ffn_dim", "in_ch",
                                    "out_ch", "frames", "height", "width", "motion_frames",
                                    "audio_per_frame", "freq_dim", "eps", "rope_theta")}
    d["cross_full"] = int(c.cross_full)
    d.update(kw)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64, n_heads=24), fh.FH_EUNSUPPORTED),
    (dict(n_heads=11), fh.FH_ESHAPE),
    (dict(motion_frames=5), fh.FH_ESHAPE),
    (dict(out_ch=8), fh.FH_ESHAPE),
    (dict(height=15), fh.FH_EUNSUPPORTED),
    (dict(audio_per_frame=20), fh.FH_EUNSUPPORTED),
    (dict(ffn_dim=9000), fh.FH_EUNSUPPORTED),
    (dict(n_blocks=0), fh.FH_ESHAPE),
    (dict(eps=float("nan")), fh.FH_ESHAPE),
    (dict(cross_full=2), fh.FH_ESHAPE),
    (dict(n_heads=3, dim=384), fh.FH_EUNSUPPORTED),     # odd head count: query sums in groups of 4
    (dict(freq_dim=2056), fh.FH_EUNSUPPORTED),          # 8 GEMV rows of it must fit 64 KiB of LDS
])
def test_create_rejects(kw, status):
    with pytest.raises(fh.FHError) as e:
        fh.fh_create(cfg_dict(**kw))
    assert e.value.status == status


def test_create_accepts_workloads():
    for name in synth.CONFIGS:
        fh.fh_create(synth.CONFIGS[name])
    fh.fh_create(cfg_dict(freq_dim=2048))
    fh.fh_create(cfg_dict(n_heads=2, dim=256))
    fh.fh_create(synth.CONFIGS["slice"].replace(cross_full=True))


def test_weight_specs_match_generator():
    for name in ("toy", "slice"):
        cfg = synth.CONFIGS[name]
        ctx = fh.fh_create(cfg)
        got = [(n, s) for n, _, s in fh.fh_weight_specs(ctx)]
        exp = [(n, tuple(s)) for n, s, _ in synth.param_specs(cfg)]
        assert sorted(got) == sorted(exp)
        kinds = {n: k for n, _, k in synth.param_specs(cfg)}
        for n, dt, _ in fh.fh_weight_specs(ctx):
            assert dt == (fh.FH_DTYPE_BF16 if kinds[n] == "matrix" else fh.FH_DTYPE_F32), n


def test_workspace_bytes():
    ctx = fh.fh_create(synth.CONFIGS["slice"])
    b1, b3 = fh.fh_workspace_bytes(ctx, 1), fh.fh_workspace_bytes(ctx, 3)
    assert b1 > 50e6 and b3 > 2.5 * b1
    assert fh.fh_workspace_bytes(ctx, 0) == 0


def _index(ctx, base_off=0, drop=None, bad_shape=None, misalign=None):
    specs = fh.fh_weight_specs(ctx)
    arr = (fh.fh_tensor * len(specs))()
    keep, off = [], base_off
    for i, (n, dt, shape) in enumerate(specs):
        nb = n.encode()
        keep.append(nb)
        arr[i].name = nb
        arr[i].dtype = dt
        arr[i].ndim = len(shape)
        for j, s in enumerate(shape):
            arr[i].shape[j] = s + (1 if n == bad_shape and j == 0 else 0)
        arr[i].offset = off + (8 if n == misalign else 0)
        off += (int(np.prod(shape)) * (2 if dt == fh.FH_DTYPE_BF16 else 4) + 255) & ~255
    n = len(specs)
    if drop is not None:
        names = [s[0] for s in specs]
        k = names.index(drop)
        arr2 = (fh.fh_tensor * (n - 1))()
        j = 0
        for i in range(n):
            if i != k:
                arr2[j] = arr[i]
                j += 1
        arr, n = arr2, n - 1
    return arr, n, off, keep


def _bind(ctx, **kw):
    arr, n, size, keep = _index(ctx, **kw)
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 40)   # never dereferenced: binding is pointer arithmetic only
    return fh.lib.fh_weights_bind(ctx, fake, size, arr, n, ctypes.byref(h)), h


def test_weights_bind_checks_index():
    ctx = fh.fh_create(synth.CONFIGS["toy"])
    st, h = _bind(ctx)
    assert st == fh.FH_OK and h.value
    fh.lib.fh_weights_release(h)
    st, _ = _bind(ctx, drop="blocks.1.ffn2.w")
    assert st == fh.FH_EWEIGHTS and "blocks.1.ffn2.w" in fh.fh_last_error(ctx)
    st, _ = _bind(ctx, bad_shape="blocks.0.qkv.w")
    assert st == fh.FH_EWEIGHTS and "shape" in fh.fh_last_error(ctx)
    st, _ = _bind(ctx, misalign="head.b")
    assert st == fh.FH_EWEIGHTS and "aligned" in fh.fh_last_error(ctx)


def test_call_argument_errors_before_any_launch():
    ctx = fh.fh_create(synth.CONFIGS["toy"])
    st, w = _bind(ctx)
    assert st == fh.FH_OK
    fake = ctypes.c_void_p(1 << 40)
    need = fh.fh_workspace_bytes(ctx, 1)
    sig = (ctypes.c_float * 2)(1.0, 0.0)
    L = fh.lib
    # batch 0, negative steps, non-finite sigma, null pointers, small or misaligned workspace
    assert L.fh_dit_denoise_slice(ctx, w, 0, fake, fake, fake, sig, 1, fake, fake, need, None) == fh.FH_EINVAL
    assert L.fh_dit_denoise_slice(ctx, w, 1, fake, fake, fake, sig, -1, fake, fake, need, None) == fh.FH_EINVAL
    bad = (ctypes.c_float * 2)(1.0, float("inf"))
    assert L.fh_dit_denoise_slice(ctx, w, 1, fake, fake, fake, bad, 1, fake, fake, need, None) == fh.FH_EINVAL
    assert "sigma" in fh.fh_last_error(ctx)
    assert L.fh_dit_denoise_slice(ctx, w, 1, None, fake, fake, sig, 1, fake, fake, need, None) == fh.FH_EINVAL
    assert L.fh_dit_denoise_slice(ctx, w, 1, fake, fake, fake, sig, 1, fake, fake, need - 1, None) == fh.FH_EWORKSPACE
    assert L.fh_dit_denoise_slice(ctx, w, 1, fake, fake, fake, sig, 1, fake,
                                  ctypes.c_void_p((1 << 40) + 64), need, None) == fh.FH_EWORKSPACE
    assert L.fh_dit_block_forward(ctx, w, 2, 1, fake, fake, fake, fake, need, None) == fh.FH_EINVAL
    assert L.fh_dit_block_forward(ctx, w, 0, 1, fake, None, fake, fake, need, None) == fh.FH_EINVAL
    assert L.fh_dit_block_forward(ctx, None, 0, 1, fake, fake, fake, fake, need, None) == fh.FH_EINVAL
    assert L.fh_set_option(ctx, 99, 0) == fh.FH_EINVAL
    assert L.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, fh.FH_K["attn"]) == fh.FH_OK
    assert L.fh_set_option(ctx, fh.FH_OPT_TIME_KERNEL, len(fh.KERNEL_CLASSES)) == fh.FH_EINVAL
    fh.lib.fh_weights_release(w)
    assert fh.fh_status_str(fh.FH_EWORKSPACE).startswith("workspace")


def test_sampler_option_and_generator_argument_errors():
    ctx = fh.fh_create(cfg_dict("toy"))
    assert fh.lib.fh_set_option(ctx, fh.FH_OPT_SAMPLER, 2) == fh.FH_EINVAL
    assert "sampler" in fh.fh_last_error(ctx)
    assert fh.lib.fh_set_option(ctx, fh.FH_OPT_SAMPLER, fh.FH_SAMPLER_RENOISE) == fh.FH_OK
    assert fh.lib.fh_set_noise_seed(ctx, 2**64 - 1) == fh.FH_OK
    assert fh.lib.fh_set_noise_seed(None, 1) == fh.FH_EINVAL
    vp = ctypes.c_void_p
    # argument checks happen before any launch: no GPU needed
    assert fh.lib.fh_philox4x32_fill(1, 0, 0, 0, 4, None, None) == fh.FH_EINVAL           # null out
    assert fh.lib.fh_philox4x32_fill(1, 0, 0, 0, 4, vp(1 << 40 | 4), None) == fh.FH_EINVAL  # misaligned
    assert fh.lib.fh_philox4x32_fill(1, 0, 0, 0, -1, vp(1 << 40), None) == fh.FH_EINVAL     # negative
    assert fh.lib.fh_philox4x32_fill(1, 0, 0, 2**32 - 2, 3, vp(1 << 40), None) == fh.FH_EINVAL  # past 2^32
    assert fh.lib.fh_philox4x32_fill(1, 0, 0, 0, 0, None, None) == fh.FH_OK                # nothing to do


def test_fp8_precision_argument_errors():
    ctx = fh.fh_create(synth.CONFIGS["toy"])
    st, w = _bind(ctx)
    assert st == fh.FH_OK
    L, vp = fh.lib, ctypes.c_void_p
    c = synth.CONFIGS["toy"]
    r = lambda b: (b + 255) // 256 * 256
    per = (r(c.ffn_dim * c.dim) * 2 + r(c.dim // 64 * c.ffn_dim * 2) + r(c.ffn_dim // 64 * c.dim * 2)
           + r(3 * c.dim * c.dim) + r(c.dim // 64 * 3 * c.dim * 2))   # FFN and QKV codes + scales
    assert fh.fh_fp8_weight_bytes(ctx) == per * c.n_blocks
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, 7) == fh.FH_EINVAL
    assert L.fh_set_option(ctx, fh.FH_OPT_PREFETCH, 0) == fh.FH_OK
    assert L.fh_set_option(ctx, fh.FH_OPT_PREFETCH, 1) == fh.FH_OK
    assert L.fh_set_option(ctx, 99, 0) == fh.FH_EINVAL
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, fh.FH_PREC_FP8_FFN) == fh.FH_OK
    # FP8 asked for before quantised weights exist: rejected before any launch
    fake = vp(1 << 40)
    need = fh.fh_workspace_bytes(ctx, 1)
    sig = (ctypes.c_float * 2)(1.0, 0.0)
    assert L.fh_dit_denoise_slice(ctx, w, 1, fake, fake, fake, sig, 1, fake, fake, need, None) == fh.FH_EINVAL
    assert "fh_weights_quantize_fp8" in fh.fh_last_error(ctx)
    assert L.fh_dit_block_forward(ctx, w, 0, 1, fake, fake, fake, fake, need, None) == fh.FH_EINVAL
    # the FP8 QKV precision: FP8 FFN's workspace, and the same need for quantised weights
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, fh.FH_PREC_FP8_QKV) == fh.FH_OK
    assert fh.fh_workspace_bytes(ctx, 1) == need
    assert L.fh_dit_denoise_slice(ctx, w, 1, fake, fake, fake, sig, 1, fake, fake, need, None) == fh.FH_EINVAL
    assert "fh_weights_quantize_fp8" in fh.fh_last_error(ctx)
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, fh.FH_PREC_FP8_FFN) == fh.FH_OK
    # quantisation buffer checks
    nb = fh.fh_fp8_weight_bytes(ctx)
    assert L.fh_weights_quantize_fp8(ctx, w, None, nb, None) == fh.FH_EINVAL
    assert L.fh_weights_quantize_fp8(ctx, w, vp((1 << 40) + 16), nb, None) == fh.FH_EINVAL   # misaligned
    assert L.fh_weights_quantize_fp8(ctx, w, fake, nb - 1, None) == fh.FH_EINVAL              # short
    assert "smaller" in fh.fh_last_error(ctx)
    # quantiser argument checks
    assert L.fh_mxfp8_quantize(fake, 4, 96, fake, fake, None) == fh.FH_EINVAL    # K not a multiple of 64
    assert L.fh_mxfp8_quantize(None, 4, 64, fake, fake, None) == fh.FH_EINVAL
    assert L.fh_mxfp8_quantize(vp((1 << 40) + 4), 4, 64, fake, fake, None) == fh.FH_EINVAL
    assert L.fh_mxfp8_quantize(fake, 0, 64, None, None, None) == fh.FH_OK
    fh.lib.fh_weights_release(w)


def test_mxfp8_gemm_argument_errors():
    """Every rejected case returns FH_EINVAL before any launch."""
    L, vp = fh.lib, ctypes.c_void_p
    f = vp(1 << 40)                       # 256-aligned stand-in device address (never touched)
    mis16, mis4 = vp((1 << 40) + 8), vp((1 << 40) + 2)

    def call(a=f, sa=f, w=f, sw=f, M=64, N=128, K=64, bias=f, y=f, part=None):
        return L.fh_mxfp8_gemm(a, sa, w, sw, M, N, K, bias, y, part, None)

    assert call(M=63) == fh.FH_EINVAL                        # M odd
    assert call(M=-2) == fh.FH_EINVAL
    assert call(N=192) == fh.FH_EINVAL                       # N % 128
    assert call(N=0) == fh.FH_EINVAL
    assert call(K=96) == fh.FH_EINVAL                        # K % 64
    for kw in ({"a": None}, {"sa": None}, {"w": None}, {"sw": None}, {"bias": None}, {"y": None}):
        assert call(**kw) == fh.FH_EINVAL, kw
    for kw in ({"a": mis16}, {"w": mis16}, {"bias": mis16}, {"y": mis16}, {"part": mis16},
               {"sa": mis4}, {"sw": mis4}):
        assert call(**kw) == fh.FH_EINVAL, kw
    assert call(part=f, K=2048) == fh.FH_EINVAL              # split needs K >= 4096
    assert call(part=f, M=1538, K=4096) == fh.FH_EINVAL      # and M <= 1536
    assert call(part=f, N=2176, K=4096) == fh.FH_EINVAL      # and N <= 2048
    assert call(M=0, a=None, y=None) == fh.FH_OK             # empty: nothing to do


def test_fp32_precision_option_and_workspace():
    ctx = fh.fh_create(synth.CONFIGS["toy"])
    L = fh.lib
    base = fh.fh_workspace_bytes(ctx, 1)
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, 5) == fh.FH_EINVAL
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, fh.FH_PREC_FP32) == fh.FH_OK
    c = synth.CONFIGS["toy"]
    N, D, Fd, La = c.frames * c.height * c.width, c.dim, c.ffn_dim, c.frames * c.audio_per_frame
    r = lambda b: (b + 255) // 256 * 256
    # float32 h, qkv, attention output, cross query, FFN hidden, audio K and V of every block
    extra = 3 * r(N * D * 4) + r(N * 3 * D * 4) + r(N * Fd * 4) + 2 * r(c.n_blocks * La * D * 4)
    assert fh.fh_workspace_bytes(ctx, 1) == base + extra
    # a workspace sized for bf16 is refused under FP32, before any launch
    st, w = _bind(ctx)
    assert st == fh.FH_OK
    fake = ctypes.c_void_p(1 << 40)
    sig = (ctypes.c_float * 2)(1.0, 0.0)
    assert L.fh_dit_denoise_slice(ctx, w, 1, fake, fake, fake, sig, 1, fake, fake, base, None) == fh.FH_EWORKSPACE
    assert L.fh_dit_block_forward(ctx, w, 0, 1, fake, fake, fake, fake, base, None) == fh.FH_EWORKSPACE
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, fh.FH_PREC_BF16) == fh.FH_OK
    assert fh.fh_workspace_bytes(ctx, 1) == base
    fh.lib.fh_weights_release(w)


def test_audio_projection_specs_and_argument_errors():
    ctx = fh.fh_create(synth.CONFIGS["toy"])
    acfg = synth.AUDIO_CONFIGS["toy"]
    specs = fh.fh_audio_weight_specs(ctx, acfg)
    want = [(n, fh.FH_DTYPE_BF16 if k == "matrix" else fh.FH_DTYPE_F32, shape)
            for n, shape, k in synth.audio_param_specs(acfg)]
    assert specs == want
    L, vp = fh.lib, ctypes.c_void_p
    bad = fh.audio_config_struct(acfg.replace(hidden=100))          # not a multiple of 128
    assert L.fh_audio_weight_count(ctx, ctypes.byref(bad)) == 0
    assert L.fh_audio_weight_count(ctx, None) == 0
    t = fh.fh_tensor()
    assert L.fh_audio_weight_spec(ctx, ctypes.byref(bad), 0, ctypes.byref(t)) == fh.FH_EINVAL
    good = fh.audio_config_struct(acfg)
    assert L.fh_audio_weight_spec(ctx, ctypes.byref(good), 10, ctypes.byref(t)) == fh.FH_EINVAL
    # binding checks need no device memory: stand-in addresses, a full and a broken index
    def index(skip=None, shape_fix=None):
        ents = [(n, d, s) for n, d, s in specs if n != skip]
        arr = (fh.fh_tensor * len(ents))()
        keep = []
        off = 0
        for i, (n, d, s) in enumerate(ents):
            nb = n.encode()
            keep.append(nb)
            arr[i].name, arr[i].dtype, arr[i].ndim = nb, d, len(s)
            for j, v in enumerate(shape_fix(n, s) if shape_fix else s):
                arr[i].shape[j] = v
            arr[i].offset = off
            off += (int(np.prod(s)) * (2 if d == fh.FH_DTYPE_BF16 else 4) + 255) // 256 * 256
        return arr, off, keep
    h = vp()
    arr, size, keep = index()
    blob = vp(1 << 40)
    assert L.fh_audio_weights_bind(ctx, ctypes.byref(bad), blob, size, arr, len(arr), ctypes.byref(h)) == \
        fh.FH_EUNSUPPORTED
    arr2, _, keep2 = index(skip="proj2.b")
    assert L.fh_audio_weights_bind(ctx, ctypes.byref(good), blob, size, arr2, len(arr2), ctypes.byref(h)) == \
        fh.FH_EWEIGHTS
    assert "proj2.b" in fh.fh_last_error(ctx)
    arr3, _, keep3 = index(shape_fix=lambda n, s: (s[0] + 1,) + s[1:] if n == "proj3.w" else s)
    assert L.fh_audio_weights_bind(ctx, ctypes.byref(good), blob, size, arr3, len(arr3), ctypes.byref(h)) == \
        fh.FH_EWEIGHTS
    assert L.fh_audio_weights_bind(ctx, ctypes.byref(good), blob, size - 256, arr, len(arr), ctypes.byref(h)) == \
        fh.FH_EWEIGHTS                                            # the last tensor outside the blob
    assert L.fh_audio_weights_bind(ctx, ctypes.byref(good), blob, size, arr, len(arr), ctypes.byref(h)) == fh.FH_OK
    need = L.fh_audio_workspace_bytes(h, 2)
    assert need > 0 and L.fh_audio_workspace_bytes(h, 0) == 0
    fake = vp(1 << 40)
    assert L.fh_audio_project(ctx, h, 2, None, fake, fake, need, None) == fh.FH_EINVAL
    assert L.fh_audio_project(ctx, h, 0, fake, fake, fake, need, None) == fh.FH_EINVAL
    assert L.fh_audio_project(ctx, h, 2, fake, fake, fake, need - 1, None) == fh.FH_EWORKSPACE
    assert L.fh_audio_project(ctx, h, 2, fake, fake, vp((1 << 40) + 16), need, None) == fh.FH_EWORKSPACE
    ctx2 = fh.fh_create(synth.CONFIGS["toy"])
    assert L.fh_audio_project(ctx2, h, 2, fake, fake, fake, need, None) == fh.FH_EINVAL   # foreign weights
    L.fh_audio_weights_release(h)


def test_fp8_attention_precision_checks():
    ctx = fh.fh_create(synth.CONFIGS["toy"])
    L = fh.lib
    base = fh.fh_workspace_bytes(ctx, 1)
    assert L.fh_set_option(ctx, fh.FH_OPT_PRECISION, fh.FH_PREC_FP8_ATTN) == fh.FH_OK
    c = synth.CONFIGS["toy"]
    N, D = c.frames * c.height * c.width, c.dim
    r = lambda b: (b + 255) // 256 * 256
    assert fh.fh_workspace_bytes(ctx, 1) == base + r(N * 2 * D) + r(N * 2 * D // 32) + r(D * N) + r(N // 64 * D * 2)
    # tokens per lane not a multiple of 64: refused before any launch
    ragged = synth.CONFIGS["slice"].replace(n_blocks=1, width=10)      # 800 tokens
    ctx2 = fh.fh_create(ragged)
    st, w = _bind(ctx2)
    assert st == fh.FH_OK
    assert L.fh_set_option(ctx2, fh.FH_OPT_PRECISION, fh.FH_PREC_FP8_ATTN) == fh.FH_OK
    fake = ctypes.c_void_p(1 << 40)
    need = fh.fh_workspace_bytes(ctx2, 1)
    sig = (ctypes.c_float * 2)(1.0, 0.0)
    assert L.fh_dit_denoise_slice(ctx2, w, 1, fake, fake, fake, sig, 1, fake, fake, need, None) == fh.FH_EUNSUPPORTED
    assert "multiple of 64" in fh.fh_last_error(ctx2)
    assert L.fh_dit_block_forward(ctx2, w, 0, 1, fake, fake, fake, fake, need, None) == fh.FH_EUNSUPPORTED
    fh.lib.fh_weights_release(w)


def test_debug_runtime_compiles():
    """The FH_DEBUG runtime (a device synchronisation after every HIP call, no
    graph capture) still compiles: syntax-only pass over its source."""
    import importlib.util
    import subprocess
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "audio_driven_talking_amd", "build.py")
    spec = importlib.util.spec_from_file_location("fh_build_check", path)
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    cmd = [b.HIPCC, *b.FLAGS, "-DFH_DEBUG", "-fsyntax-only", os.path.join(b.CSRC, "fh_api.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]


def test_color_match_workspace_and_argument_errors():
    W = fh.fh_color_match_workspace_bytes
    # (F + 1) chunks of 2048 pixels x 6 float64 sums, rounded to 256 bytes, then 9 floats per frame
    chunks = (512 * 512 + 2047) // 2048
    assert W(33, 512, 512, 512, 512) == ((34 * chunks * 48 + 255) // 256) * 256 + 33 * 36
    assert W(5, 24, 40, 7, 300) == ((6 * 2 * 48 + 255) // 256) * 256 + 5 * 36   # the picture sets the chunks
    assert W(0, 4, 4, 4, 4) == 0 and W(-1, 4, 4, 4, 4) == 0 and W(65535, 4, 4, 4, 4) == 0
    assert W(1, 0, 4, 4, 4) == 0 and W(1, 4, 4, 4, -4) == 0
    assert W(16384, 512, 512, 4, 4) == 0 and W(16383, 512, 512, 4, 4) > 0   # 2^32 - 256 frame pixels at most
    L, vp = fh.lib, ctypes.c_void_p
    a, b, o, ws = vp(1 << 40), vp((1 << 40) + (1 << 30)), vp((1 << 40) + (2 << 30)), vp((1 << 40) + (3 << 30))
    need = W(2, 8, 8, 8, 8)
    call = lambda fr, F, H, Wd, pic, s, out, w, nb: L.fh_color_match(fr, F, H, Wd, pic, 8, 8, s, out, w, nb, None)
    assert call(None, 0, 8, 8, None, 1.0, None, None, 0) == fh.FH_OK               # nothing to do
    assert call(a, -1, 8, 8, b, 1.0, o, ws, need) == fh.FH_EINVAL
    assert call(a, 2, 0, 8, b, 1.0, o, ws, need) == fh.FH_EINVAL
    assert call(a, 2, 8, 8, b, float("nan"), o, ws, need) == fh.FH_EINVAL
    assert call(a, 2, 8, 8, b, float("inf"), o, ws, need) == fh.FH_EINVAL
    assert call(None, 2, 8, 8, b, 1.0, o, ws, need) == fh.FH_EINVAL
    assert call(a, 2, 8, 8, None, 1.0, o, ws, need) == fh.FH_EINVAL
    assert call(a, 2, 8, 8, b, 1.0, None, ws, need) == fh.FH_EINVAL
    assert call(vp((1 << 40) + 2), 2, 8, 8, b, 1.0, o, ws, need) == fh.FH_EINVAL     # misaligned frames
    assert call(a, 2, 8, 8, b, 1.0, vp((1 << 40) + 64), ws, need) == fh.FH_EINVAL   # partial overlap
    assert call(a, 2, 8, 8, b, 1.0, o, None, need) == fh.FH_EINVAL
    assert call(a, 2, 8, 8, b, 1.0, o, vp((1 << 40) + (3 << 30) + 16), need) == fh.FH_EINVAL
    assert call(a, 2, 8, 8, b, 1.0, o, ws, need - 1) == fh.FH_EWORKSPACE


def test_shader_clock_argument_errors():
    """The clock probe rejects null or short buffers and out-of-range sizes
    before any launch."""
    L, fake, mhz = fh.lib, ctypes.c_void_p(1 << 40), ctypes.c_double()
    assert L.fh_shader_clock(None, 1 << 20, 16, 100, None, ctypes.byref(mhz)) == fh.FH_EINVAL
    assert L.fh_shader_clock(fake, 1 << 20, 16, 100, None, None) == fh.FH_EINVAL
    assert L.fh_shader_clock(fake, 32 * 16 - 1, 16, 100, None, ctypes.byref(mhz)) == fh.FH_EINVAL
    assert L.fh_shader_clock(fake, 1 << 30, 0, 100, None, ctypes.byref(mhz)) == fh.FH_EINVAL
    assert L.fh_shader_clock(fake, 1 << 30, 65537, 100, None, ctypes.byref(mhz)) == fh.FH_EINVAL
    assert L.fh_shader_clock(fake, 1 << 30, 16, 0, None, ctypes.byref(mhz)) == fh.FH_EINVAL


def test_vae_specs_and_argument_errors():
    """Decoder configuration checks, tensor specs and call errors, no launch."""
    vc = synth.VAE_CONFIGS["slice"]
    specs = fh.fh_vae_weight_specs(vc)
    ref = synth.vae_param_specs(vc)
    assert [s[0] for s in specs] == [r[0] for r in ref]
    for (n, dt, shape), (_, rshape, kind) in zip(specs, ref):
        assert dt == (fh.FH_DTYPE_F16 if kind == "conv" else fh.FH_DTYPE_F32)
        assert int(np.prod(shape)) == int(np.prod(rshape))
    L = fh.lib
    for bad in (vc.replace(widths=(256, 96, 64, 32)), vc.replace(patch=2), vc.replace(latent_ch=12),
                vc.replace(frames=0), vc.replace(widths=(1024, 128, 64, 32))):
        v = fh.vae_config_struct(bad)
        assert L.fh_vae_weight_count(ctypes.byref(v)) == 0
        assert L.fh_vae_workspace_bytes(ctypes.byref(v)) == 0
    v = fh.vae_config_struct(vc)
    assert L.fh_vae_workspace_bytes(ctypes.byref(v)) > 3 * 33 * 128 * 128 * 32 * 2
    h = ctypes.c_void_p()
    assert L.fh_vae_weights_bind(ctypes.byref(v), None, 0, None, 0, ctypes.byref(h)) == fh.FH_EINVAL
    assert L.fh_vae_decode(None, ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 41), ctypes.c_void_p(1 << 42),
                           1 << 30, None) == fh.FH_EINVAL


def test_slice_from_states_argument_errors():
    """The states-fed slice rejects null or foreign audio weights, null states
    and short workspaces before any launch."""
    ctx = fh.fh_create(synth.CONFIGS["toy"])
    st, w = _bind(ctx)
    assert st == fh.FH_OK
    L, fake = fh.lib, ctypes.c_void_p(1 << 40)
    sig = (ctypes.c_float * 2)(1.0, 0.0)
    assert L.fh_slice_from_states_workspace_bytes(ctx, None, 1) == 0
    assert L.fh_dit_denoise_slice_from_states(ctx, w, None, 1, fake, fake, fake, sig, 1, fake, fake, 1 << 30,
                                              None) == fh.FH_EINVAL
    fh.lib.fh_weights_release(w)


def test_debug_workgroup_order_rejects_other_values():
    assert fh.lib.fh_debug_workgroup_order(2) == fh.FH_EINVAL
    assert fh.lib.fh_debug_workgroup_order(-1) == fh.FH_EINVAL
