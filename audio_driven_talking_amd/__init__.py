"""Python binding of libfh, the MI355X slice denoiser of SoulX-FlashHead Lite.

Thin ctypes marshalling over the C ABI declared in ``include/fh.h``: the
functions here carry the C names and pass torch tensor pointers, sizes and
the current HIP stream through; every step of the computation runs in the
library's HIP kernels. PyTorch supplies device memory and streams only.

The library must have been built (``python -m audio_driven_talking_amd.build``);
importing this package without ``libfh.so`` raises ImportError -- there is no
other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# FH_DEBUG=1: the debug build (synchronises after every launch, no graphs)
LIB_PATH = os.path.join(_HERE, "libfh_debug.so" if os.environ.get("FH_DEBUG") == "1" else "libfh.so")

FH_OK, FH_EINVAL, FH_ESHAPE, FH_EUNSUPPORTED, FH_EWORKSPACE, FH_EHIP, FH_EWEIGHTS = range(7)
FH_DTYPE_BF16, FH_DTYPE_F32, FH_DTYPE_F16 = 1, 2, 3
FH_OPT_GRAPH, FH_OPT_TIME_KERNEL, FH_OPT_SAMPLER, FH_OPT_PRECISION, FH_OPT_PREFETCH = 1, 2, 3, 4, 5
FH_SAMPLER_EULER, FH_SAMPLER_RENOISE = 0, 1
FH_PREC_BF16, FH_PREC_FP8_FFN, FH_PREC_FP32, FH_PREC_FP8_ATTN, FH_PREC_FP8_QKV = 0, 1, 2, 3, 4
KERNEL_CLASSES = ["gemm_qkv", "gemm_o", "gemm_cq", "gemm_co", "gemm_ffn1", "gemm_ffn2", "attn",
                  "cross_attn", "layernorm", "rmsnorm_rope", "audio_kv"]
FH_K = {n: i for i, n in enumerate(KERNEL_CLASSES)}

# every symbol include/fh.h declares
EXPORTS = ["fh_create", "fh_destroy", "fh_weight_count", "fh_weight_spec", "fh_weights_bind",
           "fh_weights_release", "fh_workspace_bytes", "fh_dit_block_forward",
           "fh_dit_denoise_slice", "fh_set_option", "fh_set_noise_seed", "fh_philox4x32_fill",
           "fh_fp8_weight_bytes", "fh_weights_quantize_fp8", "fh_mxfp8_quantize",
           "fh_mxfp8_gemm", "fh_audio_weight_count", "fh_audio_weight_spec", "fh_audio_weights_bind",
           "fh_audio_weights_release", "fh_audio_workspace_bytes", "fh_audio_project",
           "fh_slice_from_states_workspace_bytes", "fh_dit_denoise_slice_from_states",
           "fh_color_match_workspace_bytes", "fh_color_match", "fh_color_match_noalloc",
           "fh_color_match_noalloc_max_bytes", "fh_vae_weight_count", "fh_vae_weight_spec", "fh_vae_weights_bind",
           "fh_vae_weights_release", "fh_vae_workspace_bytes", "fh_vae_decode", "fh_kernel_time", "fh_debug_workgroup_order", "fh_shader_clock",
           "fh_last_error", "fh_status_str"]


class fh_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_blocks", "dim", "n_heads", "head_dim", "ffn_dim", "in_ch", "out_ch", "frames", "height",
        "width", "motion_frames", "audio_per_frame", "freq_dim", "cross_full")] + [
        ("eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class fh_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("offset", ctypes.c_uint64)]


class fh_audio_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layers", "state_frames", "channels", "window", "temporal_stride", "hidden")]


class FHError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _load():
    # torch first: libfh must bind to the HIP runtime torch already loaded
    # (same soname), since it receives torch's device pointers and streams.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        debug = "FH_DEBUG=1 " if LIB_PATH.endswith("_debug.so") else ""
        raise ImportError(f"{LIB_PATH} is not built: run `{debug}python audio_driven_talking_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "fh_create": (i32, [ctypes.POINTER(fh_config), ctypes.POINTER(vp)]),
        "fh_destroy": (None, [vp]),
        "fh_weight_count": (i32, [vp]),
        "fh_weight_spec": (i32, [vp, i32, ctypes.POINTER(fh_tensor)]),
        "fh_weights_bind": (i32, [vp, vp, sz, ctypes.POINTER(fh_tensor), i32, ctypes.POINTER(vp)]),
        "fh_weights_release": (None, [vp]),
        "fh_workspace_bytes": (sz, [vp, i32]),
        "fh_dit_block_forward": (i32, [vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]),
        "fh_dit_denoise_slice": (i32, [vp, vp, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_float), i32,
                                       vp, vp, sz, vp]),
        "fh_set_option": (i32, [vp, i32, i32]),
        "fh_set_noise_seed": (i32, [vp, ctypes.c_uint64]),
        "fh_fp8_weight_bytes": (sz, [vp]),
        "fh_weights_quantize_fp8": (i32, [vp, vp, vp, sz, vp]),
        "fh_mxfp8_quantize": (i32, [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]),
        "fh_mxfp8_gemm": (i32, [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp]),
        "fh_audio_weight_count": (i32, [vp, vp]),
        "fh_audio_weight_spec": (i32, [vp, vp, i32, vp]),
        "fh_audio_weights_bind": (i32, [vp, vp, vp, sz, vp, i32, vp]),
        "fh_audio_weights_release": (None, [vp]),
        "fh_audio_workspace_bytes": (sz, [vp, i32]),
        "fh_audio_project": (i32, [vp, vp, i32, vp, vp, vp, sz, vp]),
        "fh_slice_from_states_workspace_bytes": (sz, [vp, vp, i32]),
        "fh_dit_denoise_slice_from_states": (i32, [vp, vp, vp, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_float), i32,
                                                   vp, vp, sz, vp]),
        "fh_philox4x32_fill": (i32, [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.c_int64, vp, vp]),
        "fh_color_match_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "fh_color_match": (i32, [vp, i32, i32, i32, vp, i32, i32, ctypes.c_float, vp, vp, sz, vp]),
        "fh_color_match_noalloc": (i32, [vp, i32, i32, i32, vp, i32, i32, ctypes.c_float, vp, vp]),
        "fh_color_match_noalloc_max_bytes": (sz, []),
        "fh_vae_weight_count": (i32, [vp]),
        "fh_vae_weight_spec": (i32, [vp, i32, ctypes.POINTER(fh_tensor)]),
        "fh_vae_weights_bind": (i32, [vp, vp, sz, ctypes.POINTER(fh_tensor), i32, ctypes.POINTER(vp)]),
        "fh_vae_weights_release": (None, [vp]),
        "fh_vae_workspace_bytes": (sz, [vp]),
        "fh_vae_decode": (i32, [vp, vp, vp, vp, sz, vp]),
        "fh_kernel_time": (i32, [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
        "fh_shader_clock": (i32, [vp, ctypes.c_size_t, i32, i32, vp, ctypes.POINTER(ctypes.c_double)]),
        "fh_debug_workgroup_order": (i32, [i32]),
        "fh_last_error": (ctypes.c_char_p, [vp]),
        "fh_status_str": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


lib = _load()


def _check(ctx, status):
    if status != FH_OK:
        msg = lib.fh_last_error(ctx).decode() if ctx else lib.fh_status_str(status).decode()
        raise FHError(status, msg or lib.fh_status_str(status).decode())


def _cfg_struct(cfg) -> fh_config:
    get = (lambda k: cfg[k]) if isinstance(cfg, dict) else (lambda k: getattr(cfg, k))
    s = fh_config()
    for n, _ in fh_config._fields_:
        v = get(n)
        setattr(s, n, float(v) if n in ("eps", "rope_theta") else int(v))
    return s


class Context:
    """An fh_ctx*. Destroyed with the object."""

    def __init__(self, handle, cfg):
        self.handle = handle
        self.cfg = cfg
        self._free = lib.fh_destroy   # kept: module globals may be gone when this object dies

    def __del__(self):
        if getattr(self, "handle", None):
            self._free(self.handle)
            self.handle = None

    @property
    def _as_parameter_(self):
        return self.handle


class Weights:
    """An fh_weights* plus the device blob it points into (kept alive here)."""

    def __init__(self, handle, blob, ctx):
        self.handle, self.blob, self.ctx = handle, blob, ctx
        self._free = lib.fh_weights_release

    def __del__(self):
        if getattr(self, "handle", None):
            self._free(self.handle)
            self.handle = None

    @property
    def _as_parameter_(self):
        return self.handle


def fh_create(cfg) -> Context:
    """cfg: a mapping or object with the fh_config field names."""
    h = ctypes.c_void_p()
    st = lib.fh_create(ctypes.byref(_cfg_struct(cfg)), ctypes.byref(h))
    if st != FH_OK:
        raise FHError(st, lib.fh_status_str(st).decode())
    return Context(h, cfg)


def fh_weight_specs(ctx: Context):
    """[(name, dtype, shape)] the context needs, in its order."""
    out = []
    t = fh_tensor()
    for i in range(lib.fh_weight_count(ctx)):
        _check(ctx, lib.fh_weight_spec(ctx, i, ctypes.byref(t)))
        out.append((t.name.decode(), t.dtype, tuple(t.shape[:t.ndim])))
    return out


def _host_bytes(a):
    """numpy uint16 (bf16 bits) / float32 array, or a torch tensor, as (bytes view, dtype code)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            t = a.detach().contiguous().cpu()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint8), FH_DTYPE_BF16
            if t.dtype == torch.float32:
                return t.numpy().view(np.uint8), FH_DTYPE_F32
            if t.dtype == torch.float16:
                return t.numpy().view(np.uint8), FH_DTYPE_F16
            raise TypeError(f"unsupported tensor dtype {t.dtype}")
    except ImportError:
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a.view(np.uint8).reshape(-1), FH_DTYPE_BF16
    if a.dtype == np.float32:
        return a.view(np.uint8).reshape(-1), FH_DTYPE_F32
    if a.dtype == np.float16:
        return a.view(np.uint8).reshape(-1), FH_DTYPE_F16
    raise TypeError(f"unsupported array dtype {a.dtype}")


def _pack_blob(specs, tensors, device):
    """One device blob holding `tensors` in `specs` order at 256-byte aligned
    offsets, and its fh_tensor index (with the name buffers kept alive)."""
    import torch
    entries, off = [], 0
    for name, _, shape in specs:
        if name not in tensors:
            raise KeyError(f"weight {name!r} missing")
        buf, code = _host_bytes(tensors[name])
        entries.append((name, code, shape, off, buf))
        off = (off + buf.size + 255) & ~255
    host = np.zeros(max(off, 256), dtype=np.uint8)
    for _, _, _, o, buf in entries:
        host[o:o + buf.size] = buf
    blob = torch.from_numpy(host).to(device)
    index = (fh_tensor * len(entries))()
    names = []
    for i, (name, code, shape, o, _) in enumerate(entries):
        nb = name.encode()
        names.append(nb)
        index[i].name = nb
        index[i].dtype = code
        index[i].ndim = len(shape)
        for j, sz in enumerate(shape):
            index[i].shape[j] = sz
        index[i].offset = o
    return blob, index, names


def fh_weights_bind(ctx: Context, tensors: dict, device="cuda") -> Weights:
    """Pack `tensors` (name -> bf16-bits uint16 / float32 arrays or tensors) into
    one device blob at 256-byte aligned offsets and bind it."""
    blob, index, _names = _pack_blob(fh_weight_specs(ctx), tensors, device)
    h = ctypes.c_void_p()
    _check(ctx, lib.fh_weights_bind(ctx, ctypes.c_void_p(blob.data_ptr()), blob.numel(), index,
                                    len(index), ctypes.byref(h)))
    return Weights(h, blob, ctx)


def fh_workspace_bytes(ctx: Context, batch: int) -> int:
    return int(lib.fh_workspace_bytes(ctx, int(batch)))


def workspace(ctx: Context, batch: int, device="cuda"):
    """A device byte tensor of fh_workspace_bytes(ctx, batch)."""
    import torch
    return torch.empty(fh_workspace_bytes(ctx, batch), dtype=torch.uint8, device=device)


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))


def _dev_f32(t, shape, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 \
            or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 device tensor of shape {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _dims(ctx):
    c = ctx.cfg
    get = (lambda k: c[k]) if isinstance(c, dict) else (lambda k: getattr(c, k))
    return {k: int(get(k)) for k in ("dim", "in_ch", "frames", "height", "width", "motion_frames",
                                     "audio_per_frame")}


def fh_dit_block_forward(ctx, w, block, x, temb, audio, ws, stream=None):
    """One DiT block in place on x [B, N, D] (device f32)."""
    d = _dims(ctx)
    B = x.shape[0]
    N, D = d["frames"] * d["height"] * d["width"], d["dim"]
    _check(ctx, lib.fh_dit_block_forward(
        ctx, w, int(block), B, _dev_f32(x, (B, N, D), "x"), _dev_f32(temb, (B, D), "temb"),
        _dev_f32(audio, (B, d["frames"] * d["audio_per_frame"], D), "audio"),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))


def fh_dit_denoise_slice(ctx, w, latent, motion_latent, audio_tokens, sigmas, latent_out, ws,
                         stream=None):
    """Denoise [B, C, F, H, W] latents with len(sigmas)-1 steps of the context's
    sampler (Euler unless FH_OPT_SAMPLER says otherwise; host sigmas)."""
    d = _dims(ctx)
    B = latent.shape[0]
    C, F, H, W = d["in_ch"], d["frames"], d["height"], d["width"]
    sig = (ctypes.c_float * max(len(sigmas), 1))(*[float(s) for s in sigmas])
    _check(ctx, lib.fh_dit_denoise_slice(
        ctx, w, B, _dev_f32(latent, (B, C, F, H, W), "latent"),
        _dev_f32(motion_latent, (B, C, d["motion_frames"], H, W), "motion_latent"),
        _dev_f32(audio_tokens, (B, F * d["audio_per_frame"], d["dim"]), "audio_tokens"),
        sig, len(sigmas) - 1, _dev_f32(latent_out, (B, C, F, H, W), "latent_out"),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))


def fh_set_option(ctx, option, value):
    _check(ctx, lib.fh_set_option(ctx, int(option), int(value)))


def fh_set_noise_seed(ctx, seed):
    _check(ctx, lib.fh_set_noise_seed(ctx, int(seed) & (2**64 - 1)))


def fh_philox4x32_fill(seed, lane, step, first_group, out, stream=None):
    """Fill the device uint32 view `out` (4 words per group, a multiple of 4
    long) with the sampler's Philox-4x32-10 words (see include/fh.h)."""
    import torch
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.element_size() != 4 \
            or not out.is_contiguous() or out.numel() % 4:
        raise ValueError("out must be a contiguous 4-byte device tensor with a multiple of 4 elements")
    st = lib.fh_philox4x32_fill(int(seed) & (2**64 - 1), int(lane), int(step), int(first_group),
                                out.numel() // 4, ctypes.c_void_p(out.data_ptr()), _stream(stream))
    if st != FH_OK:
        raise FHError(st, f"fh_philox4x32_fill: {fh_status_str(st)}")


def fh_color_match_workspace_bytes(n_frames, height, width, ref_height, ref_width):
    return int(lib.fh_color_match_workspace_bytes(n_frames, height, width, ref_height, ref_width))


def fh_color_match(frames, picture, strength=1.0, out=None, workspace=None, stream=None):
    """Lab colour match of float32 device planes frames [3, F, H, W] to
    picture [3, H', W'] (see include/fh.h). Returns out (a new tensor unless
    given; it may be frames for an in-place call)."""
    import torch
    for name, t, nd in (("frames", frames, 4), ("picture", picture, 3)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or t.dim() != nd \
                or not t.is_contiguous() or t.shape[0] != 3:
            raise ValueError(f"{name} must be a contiguous float32 device tensor [3, ...] of {nd} dims")
    _, F, H, W = frames.shape
    _, Hr, Wr = picture.shape
    if out is None:
        out = torch.empty_like(frames)
    elif out.shape != frames.shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like frames")
    if workspace is None:
        workspace = torch.empty(max(fh_color_match_workspace_bytes(F, H, W, Hr, Wr), 1), dtype=torch.uint8,
                                device=frames.device)
    st = lib.fh_color_match(ctypes.c_void_p(frames.data_ptr()), F, H, W, ctypes.c_void_p(picture.data_ptr()),
                            Hr, Wr, float(strength), ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream))
    if st != FH_OK:
        raise FHError(st, f"fh_color_match: {fh_status_str(st)}")
    return out


def fh_color_match_noalloc(frames, picture, strength=1.0, out=None, stream=None):
    """fh_color_match with its statistics in the library's static device
    scratch: no workspace argument (see include/fh.h). Returns out."""
    import torch
    for name, t, nd in (("frames", frames, 4), ("picture", picture, 3)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or t.dim() != nd \
                or not t.is_contiguous() or t.shape[0] != 3:
            raise ValueError(f"{name} must be a contiguous float32 device tensor [3, ...] of {nd} dims")
    _, F, H, W = frames.shape
    _, Hr, Wr = picture.shape
    if out is None:
        out = torch.empty_like(frames)
    elif out.shape != frames.shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like frames")
    st = lib.fh_color_match_noalloc(ctypes.c_void_p(frames.data_ptr()), F, H, W, ctypes.c_void_p(picture.data_ptr()),
                                    Hr, Wr, float(strength), ctypes.c_void_p(out.data_ptr()), _stream(stream))
    if st != FH_OK:
        raise FHError(st, f"fh_color_match_noalloc: {fh_status_str(st)}")
    return out


def fh_fp8_weight_bytes(ctx):
    return int(lib.fh_fp8_weight_bytes(ctx))


def fh_weights_quantize_fp8(ctx, w, stream=None, device="cuda"):
    """Quantise w's FFN and QKV matrices to MX-FP8 into a new device buffer kept on w."""
    import torch
    buf = torch.empty(fh_fp8_weight_bytes(ctx) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    _check(ctx, lib.fh_weights_quantize_fp8(ctx, w, ctypes.c_void_p(buf.data_ptr() + off),
                                            buf.numel() - off, _stream(stream)))
    w.fp8_buffer = buf


def fh_mxfp8_quantize(x, stream=None):
    """MX-FP8 codes [rows, K] (uint8) and scales [K/64, rows] (int16 bit patterns)
    of a contiguous float32 device tensor [rows, K]."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != torch.float32 or x.dim() != 2 \
            or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float32 device tensor")
    rows, K = x.shape
    codes = torch.empty(rows, K, dtype=torch.uint8, device=x.device)
    scales = torch.empty(K // 64 if K % 64 == 0 else 0, rows, dtype=torch.int16, device=x.device)
    st = lib.fh_mxfp8_quantize(ctypes.c_void_p(x.data_ptr()), rows, K, ctypes.c_void_p(codes.data_ptr()),
                               ctypes.c_void_p(scales.data_ptr()), _stream(stream))
    if st != FH_OK:
        raise FHError(st, f"fh_mxfp8_quantize: {fh_status_str(st)}")
    return codes, scales


def fh_mxfp8_gemm(a_codes, a_scales, w_codes, w_scales, bias, y, part=None, stream=None):
    """y += dec(A) dec(W)^T + bias (float32, in place) from MX-FP8 codes and
    scales as fh_mxfp8_quantize returns them; with `part` (float32, 2*M*N
    elements) K is split in two halves."""
    import torch
    M, K = a_codes.shape
    N = w_codes.shape[0]
    for t, dt in ((a_codes, torch.uint8), (w_codes, torch.uint8), (a_scales, torch.int16),
                  (w_scales, torch.int16), (bias, torch.float32), (y, torch.float32)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dt or not t.is_contiguous():
            raise ValueError("operands must be contiguous device tensors of the documented dtypes")
    if w_codes.shape[1] != K or tuple(y.shape) != (M, N) or bias.numel() != N:
        raise ValueError("shape mismatch")
    if part is not None and (part.dtype != torch.float32 or part.numel() < 2 * M * N):
        raise ValueError("part must hold 2*M*N float32")
    p = ctypes.c_void_p(part.data_ptr()) if part is not None else None
    st = lib.fh_mxfp8_gemm(ctypes.c_void_p(a_codes.data_ptr()), ctypes.c_void_p(a_scales.data_ptr()),
                           ctypes.c_void_p(w_codes.data_ptr()), ctypes.c_void_p(w_scales.data_ptr()),
                           M, N, K, ctypes.c_void_p(bias.data_ptr()), ctypes.c_void_p(y.data_ptr()), p,
                           _stream(stream))
    if st != FH_OK:
        raise FHError(st, f"fh_mxfp8_gemm: {fh_status_str(st)}")
    return y


def fh_kernel_time(ctx):
    """(total ms, launches) of the timed kernel class since the last read."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(ctx, lib.fh_kernel_time(ctx, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def fh_shader_clock(n_wg=1024, iters=20000, stream=None):
    """Median shader clock (MHz) of n_wg workgroups running back-to-back bf16
    MFMAs (a measurement aid; waits for the probe)."""
    import torch
    buf = torch.empty(32 * n_wg, dtype=torch.uint8, device="cuda")
    mhz = ctypes.c_double()
    st = lib.fh_shader_clock(ctypes.c_void_p(buf.data_ptr()), buf.numel(), int(n_wg), int(iters), _stream(stream),
                             ctypes.byref(mhz))
    if st != FH_OK:
        raise FHError(st, f"fh_shader_clock: {fh_status_str(st)}")
    return mhz.value


def fh_debug_workgroup_order(reversed_order: bool):
    """Reverse (True) or restore the workgroup order of the LDS-sharing kernels."""
    st = lib.fh_debug_workgroup_order(int(bool(reversed_order)))
    if st != FH_OK:
        raise FHError(st, f"fh_debug_workgroup_order: {fh_status_str(st)}")


def fh_last_error(ctx):
    return lib.fh_last_error(ctx).decode()


def fh_status_str(status):
    return lib.fh_status_str(int(status)).decode()


# ---------------------------------------------------------------- audio projection front end
def audio_config_struct(acfg) -> fh_audio_config:
    """fh_audio_config from a mapping or an object with the same field names."""
    get = (lambda k: acfg[k]) if isinstance(acfg, dict) else (lambda k: getattr(acfg, k))
    c = fh_audio_config()
    for n, _ in fh_audio_config._fields_:
        setattr(c, n, int(get(n)))
    return c


class AudioWeights:
    """An fh_audio_weights* plus its device blob and configuration (kept alive here)."""

    def __init__(self, handle, blob, ctx, acfg):
        self.handle, self.blob, self.ctx, self.acfg = handle, blob, ctx, acfg
        self._free = lib.fh_audio_weights_release

    def __del__(self):
        if getattr(self, "handle", None):
            self._free(self.handle)
            self.handle = None

    @property
    def _as_parameter_(self):
        return self.handle


def fh_audio_weight_specs(ctx: Context, acfg):
    """[(name, dtype, shape)] of the front end's tensors for `acfg` on this context."""
    a = audio_config_struct(acfg)
    n = lib.fh_audio_weight_count(ctx, ctypes.byref(a))
    if n <= 0:
        raise FHError(FH_EINVAL, "invalid audio configuration")
    out, t = [], fh_tensor()
    for i in range(n):
        _check(None, lib.fh_audio_weight_spec(ctx, ctypes.byref(a), i, ctypes.byref(t)))
        out.append((t.name.decode(), t.dtype, tuple(t.shape[:t.ndim])))
    return out


def fh_audio_weights_bind(ctx: Context, acfg, tensors: dict, device="cuda") -> AudioWeights:
    a = audio_config_struct(acfg)
    blob, index, _names = _pack_blob(fh_audio_weight_specs(ctx, acfg), tensors, device)
    h = ctypes.c_void_p()
    _check(ctx, lib.fh_audio_weights_bind(ctx, ctypes.byref(a), ctypes.c_void_p(blob.data_ptr()), blob.numel(),
                                          index, len(index), ctypes.byref(h)))
    return AudioWeights(h, blob, ctx, a)


def fh_audio_workspace_bytes(aw: AudioWeights, batch: int) -> int:
    return int(lib.fh_audio_workspace_bytes(aw, int(batch)))


def audio_workspace(aw: AudioWeights, batch: int, device="cuda"):
    import torch
    return torch.empty(fh_audio_workspace_bytes(aw, batch), dtype=torch.uint8, device=device)


def fh_audio_project(ctx, aw, states, tokens, ws, stream=None):
    """states [B, layers, state_frames, channels] -> tokens [B, frames * audio_per_frame, dim]
    (float32 device tensors; `tokens` written)."""
    d = _dims(ctx)
    a = aw.acfg
    B = states.shape[0]
    _check(ctx, lib.fh_audio_project(
        ctx, aw, B, _dev_f32(states, (B, a.layers, a.state_frames, a.channels), "states"),
        _dev_f32(tokens, (B, d["frames"] * d["audio_per_frame"], d["dim"]), "tokens"),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))


def fh_slice_from_states_workspace_bytes(ctx, aw, batch: int) -> int:
    return int(lib.fh_slice_from_states_workspace_bytes(ctx, aw, int(batch)))


def slice_from_states_workspace(ctx, aw, batch: int, device="cuda"):
    import torch
    return torch.empty(fh_slice_from_states_workspace_bytes(ctx, aw, batch), dtype=torch.uint8, device=device)


def fh_dit_denoise_slice_from_states(ctx, w, aw, latent, motion_latent, states, sigmas, latent_out, ws,
                                     stream=None):
    """The slice denoise fed from speech-encoder states [B, layers, state_frames,
    channels] (the audio projection front end inside the same call)."""
    d = _dims(ctx)
    a = aw.acfg
    B = latent.shape[0]
    C, F, H, W = d["in_ch"], d["frames"], d["height"], d["width"]
    sig = (ctypes.c_float * max(len(sigmas), 1))(*[float(s) for s in sigmas])
    _check(ctx, lib.fh_dit_denoise_slice_from_states(
        ctx, w, aw, B, _dev_f32(latent, (B, C, F, H, W), "latent"),
        _dev_f32(motion_latent, (B, C, d["motion_frames"], H, W), "motion_latent"),
        _dev_f32(states, (B, a.layers, a.state_frames, a.channels), "states"),
        sig, len(sigmas) - 1, _dev_f32(latent_out, (B, C, F, H, W), "latent_out"),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))


# ---------------------------------------------------------------- video decoder
class fh_vae_config(ctypes.Structure):
    _fields_ = [("latent_ch", ctypes.c_int32), ("frames", ctypes.c_int32), ("height", ctypes.c_int32),
                ("width", ctypes.c_int32), ("widths", ctypes.c_int32 * 4), ("out_ch", ctypes.c_int32),
                ("patch", ctypes.c_int32), ("eps", ctypes.c_float)]


def vae_config_struct(vc):
    """fh_vae_config from an object with the same fields (e.g. synth.VaeConfig)."""
    if isinstance(vc, fh_vae_config):
        return vc
    return fh_vae_config(vc.latent_ch, vc.frames, vc.height, vc.width, (ctypes.c_int32 * 4)(*vc.widths),
                         vc.out_ch, vc.patch, vc.eps)


class VaeWeights:
    """An fh_vae_weights* plus its device blob and configuration (kept alive here)."""

    def __init__(self, handle, blob, cfg):
        self.handle, self.blob, self.cfg = handle, blob, cfg
        self._free = lib.fh_vae_weights_release

    def __del__(self):
        if getattr(self, "handle", None):
            self._free(self.handle)
            self.handle = None

    @property
    def _as_parameter_(self):
        return self.handle


def fh_vae_weight_specs(vc):
    """[(name, dtype, shape)] of a decoder's tensors."""
    v = vae_config_struct(vc)
    n = lib.fh_vae_weight_count(ctypes.byref(v))
    if n <= 0:
        raise FHError(FH_EINVAL, "unsupported decoder configuration")
    out, t = [], fh_tensor()
    for i in range(n):
        _check(None, lib.fh_vae_weight_spec(ctypes.byref(v), i, ctypes.byref(t)))
        out.append((t.name.decode(), t.dtype, tuple(t.shape[:t.ndim])))
    return out


def fh_vae_weights_bind(vc, tensors: dict, device="cuda") -> VaeWeights:
    """Pack the decoder's tensors (kernels as float16 arrays, or uint16 arrays of
    float16 bits, any shape of the right size; biases and gains float32) into
    one device blob and bind it."""
    v = vae_config_struct(vc)
    ts = {k: (a.view(np.float16) if isinstance(a, np.ndarray) and a.dtype == np.uint16 else a)
          for k, a in tensors.items()}
    blob, index, _names = _pack_blob(fh_vae_weight_specs(v), ts, device)
    h = ctypes.c_void_p()
    _check(None, lib.fh_vae_weights_bind(ctypes.byref(v), ctypes.c_void_p(blob.data_ptr()), blob.numel(), index,
                                         len(index), ctypes.byref(h)))
    return VaeWeights(h, blob, v)


def fh_vae_workspace_bytes(vc) -> int:
    return int(lib.fh_vae_workspace_bytes(ctypes.byref(vae_config_struct(vc))))


def fh_vae_decode(vw: VaeWeights, latent, frames=None, workspace=None, stream=None):
    """Decode a float32 device latent [latent_ch, F, H, W] to frames
    [out_ch, 8 (F - 1) + 1, 32 H, 32 W] in [0, 1] (see include/fh.h)."""
    import torch
    v = vw.cfg
    shape = (v.latent_ch, v.frames, v.height, v.width)
    out_shape = (v.out_ch, 8 * (v.frames - 1) + 1, 8 * v.patch * v.height, 8 * v.patch * v.width)
    if not isinstance(latent, torch.Tensor) or not latent.is_cuda or latent.dtype != torch.float32 \
            or not latent.is_contiguous() or tuple(latent.shape) != shape:
        raise ValueError(f"latent must be a contiguous float32 device tensor of shape {shape}")
    if frames is None:
        frames = torch.empty(out_shape, dtype=torch.float32, device=latent.device)
    elif tuple(frames.shape) != out_shape or frames.dtype != torch.float32 or not frames.is_contiguous():
        raise ValueError(f"frames must be a contiguous float32 tensor of shape {out_shape}")
    if workspace is None:
        workspace = torch.empty(fh_vae_workspace_bytes(v), dtype=torch.uint8, device=latent.device)
    st = lib.fh_vae_decode(vw, ctypes.c_void_p(latent.data_ptr()), ctypes.c_void_p(frames.data_ptr()),
                           ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream))
    if st != FH_OK:
        raise FHError(st, f"fh_vae_decode: {fh_status_str(st)}")
    return frames
