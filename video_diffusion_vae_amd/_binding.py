"""ctypes binding of libvae_mi355x.so: the same entry points as include/vae.h.

Argument marshalling only. Torch tensors supply device memory and the current HIP stream. Every
step of the decode runs in the library's HIP kernels, and there is no Python or CPU fallback: if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

# VAE_MI355X_LIB points at another build of the library (e.g. the sanitized host build).
LIB_PATH = os.environ.get("VAE_MI355X_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libvae_mi355x.so")

VAE_OK, VAE_ERR_INVALID_ARG, VAE_ERR_UNSUPPORTED, VAE_ERR_HIP, VAE_ERR_WORKSPACE = range(5)
VAE_DTYPE_BF16, VAE_DTYPE_F32, VAE_DTYPE_F16 = 1, 2, 3
VAE_UPSAMPLE_NEAREST, VAE_UPSAMPLE_D2S = 1, 2
VAE_TILING_PATCH_HALO, VAE_TILING_OVERLAP_BLEND = 1, 2
VAE_LAUNCH_MERGED, VAE_LAUNCH_PER_PATCH = 0, 1
VAE_STATUS_NONFINITE = 1
VAE_MERGE_ZERO, VAE_MERGE_FINALIZE = 1, 2
VAE_CONV_SPLIT_FP32, VAE_CONV_PACKED_WEIGHTS, VAE_CONV_PACKED_F16_WEIGHTS = 1, 2, 4
VAE_CONV_SPLIT_K = 8
VAE_DECODE_SPLIT_FP32_OPERANDS, VAE_DECODE_F16_OPERANDS, VAE_DECODE_NORM_IN_CONV = 1, 2, 4
VAE_OP_CONV, VAE_OP_RES, VAE_OP_GN_SILU, VAE_OP_D2S, VAE_OP_NEAREST = 1, 2, 3, 4, 5
VAE_OP_RES_RMS, VAE_OP_RMS_SILU, VAE_OP_ATTN, VAE_OP_S2D, VAE_OP_CONV_DOWN = 6, 7, 8, 9, 10
VAE_PAD_AROUND, VAE_PAD_AFTER = 0, 1
PAD_CODES = {"around": VAE_PAD_AROUND, "after": VAE_PAD_AFTER}
VAE_KIND_NAMES = {1: "conv", 2: "gn", 3: "upsample", 4: "merge", 5: "other", 6: "rms", 7: "attn"}

# Every symbol include/vae.h declares.
EXPORTS = (
    "vae_last_error", "vae_last_error_info", "vae_version", "vae_conv3d_causal",
    "vae_conv3d_causal_strided",
    "vae_conv3d_causal_fused_workspace", "vae_conv3d_causal_fused", "vae_conv_weight_pack_size", "vae_conv_weight_pack", "vae_conv_weight_pack_f16",
    "vae_decoder_packed_weight_size",
    "vae_decoder_pack_weights",
    "vae_groupnorm_silu_workspace", "vae_groupnorm_silu", "vae_groupnorm_silu_noalloc",
    "vae_groupnorm_stats_workspace",
    "vae_groupnorm_stats", "vae_groupnorm_combine", "vae_groupnorm_apply",
    "vae_groupnorm_scale_shift", "vae_rmsnorm_silu",
    "vae_frame_attention_workspace", "vae_frame_attention", "vae_upsample", "vae_space_to_depth",
    "vae_tile_split", "vae_tile_merge", "vae_decoder_create", "vae_decoder_destroy",
    "vae_decoder_set_launch", "vae_decoder_set_clip_frames", "vae_decode_workspace_size",
    "vae_decode_tiled",
    "vae_decode_status",
    "vae_decoder_set_timing",
    "vae_decoder_get_timing",
)


class vae_tensor_t(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n", ctypes.c_int64), ("t", ctypes.c_int64), ("h", ctypes.c_int64),
                ("w", ctypes.c_int64), ("c", ctypes.c_int64)]


class vae_box_t(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("t0", "t1", "h0", "h1", "w0", "w1")]



class vae_conv_fused_t(ctypes.Structure):
    _fields_ = [("x", ctypes.POINTER(vae_tensor_t)), ("weight", ctypes.c_void_p),
                ("weight_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("bias", ctypes.c_void_p), ("residual", ctypes.POINTER(vae_tensor_t)),
                ("y", ctypes.POINTER(vae_tensor_t)), ("out_box", ctypes.POINTER(vae_box_t)),
                ("d2s_st", ctypes.c_int32), ("d2s_sh", ctypes.c_int32), ("d2s_sw", ctypes.c_int32),
                ("gn_groups", ctypes.c_int32), ("gn_eps", ctypes.c_float),
                ("gn_mean_rstd", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t), ("in_up_sh", ctypes.c_int32),
                ("in_up_sw", ctypes.c_int32), ("in_scale_shift", ctypes.c_void_p)]

class vae_error_info_t(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("axis", ctypes.c_int32), ("extent", ctypes.c_int64),
                ("required_multiple", ctypes.c_int64), ("min_width", ctypes.c_int64)]


class vae_tiling_desc_t(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in (
        "mode", "n", "t", "h", "w", "scale_t", "scale_h", "scale_w", "patches_h", "patches_w",
        "tile_h", "tile_w", "stride_h", "stride_w", "tile_t", "stride_t", "down_t", "down_h",
        "down_w")]


class vae_tile_t(ctypes.Structure):
    _fields_ = [("index", ctypes.c_int32), ("row", ctypes.c_int32), ("col", ctypes.c_int32),
                ("latent", vae_box_t), ("out", vae_box_t),
                ("lead_t", ctypes.c_int32), ("lead_h", ctypes.c_int32), ("lead_w", ctypes.c_int32),
                ("trail_t", ctypes.c_int32), ("trail_h", ctypes.c_int32),
                ("trail_w", ctypes.c_int32)]


class vae_layer_desc_t(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32)
                for k in ("op", "cin", "cout", "st", "sh", "sw", "f32_out", "no_split", "pad")]


class vae_decoder_spec_t(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("latent_channels", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("eps", ctypes.c_float), ("n_layers", ctypes.c_int32),
                ("layers", ctypes.POINTER(vae_layer_desc_t))]


class vae_op_timing_t(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python video_diffusion_vae_amd/build.py`")
    # torch first: it loads the HIP runtime that owns the device memory and streams handed to the
    # library, and the library then binds to that same runtime (one libamdhip64 per process).
    # Loaded the other way round, the device was not found on the GPU host.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    T = ctypes.POINTER(vae_tensor_t)
    B = ctypes.POINTER(vae_box_t)
    D = ctypes.POINTER(vae_tiling_desc_t)
    sig = {
        "vae_last_error": ([], ctypes.c_char_p),
        "vae_last_error_info": ([ctypes.POINTER(vae_error_info_t)], I32),
        "vae_version": ([], I32),
        "vae_conv3d_causal": ([T, P, I32, P, T, T, B, I32, P], I32),
        "vae_conv3d_causal_strided": ([T, P, I32, P, T, T, B, I32, I32, I32, I32, I32, P], I32),
        "vae_conv3d_causal_fused_workspace": ([ctypes.POINTER(vae_conv_fused_t),
                                               ctypes.POINTER(SZ)], I32),
        "vae_conv3d_causal_fused": ([ctypes.POINTER(vae_conv_fused_t), P], I32),
        "vae_conv_weight_pack_size": ([I32, I32, ctypes.POINTER(SZ)], I32),
        "vae_conv_weight_pack": ([P, I32, I32, P, P], I32),
        "vae_conv_weight_pack_f16": ([P, I32, I32, P, P], I32),
        "vae_decoder_packed_weight_size": ([P, ctypes.POINTER(SZ)], I32),
        "vae_decoder_pack_weights": ([P, P, SZ, P], I32),
        "vae_groupnorm_silu_workspace": ([T, B, I32, I32, ctypes.POINTER(SZ)], I32),
        "vae_groupnorm_silu": ([T, B, I32, I32, F, P, P, I32, T, P, SZ, P], I32),
        "vae_groupnorm_silu_noalloc": ([T, B, I32, I32, F, P, P, I32, T, P], I32),
        "vae_groupnorm_stats_workspace": ([T, B, I32, I32, ctypes.POINTER(SZ)], I32),
        "vae_groupnorm_stats": ([T, B, I32, I32, P, P, SZ, P], I32),
        "vae_groupnorm_combine": ([P, I32, I32, I32, F, P, P], I32),
        "vae_groupnorm_apply": ([T, B, I32, P, P, P, I32, T, P], I32),
        "vae_groupnorm_scale_shift": ([P, I32, I32, I32, P, P, P, P], I32),
        "vae_rmsnorm_silu": ([T, F, P, P, I32, T, P], I32),
        "vae_frame_attention_workspace": ([T, ctypes.POINTER(SZ)], I32),
        "vae_frame_attention": ([T, F, P, P, P, P, P, P, T, P, SZ, P], I32),
        "vae_upsample": ([T, B, I32, I32, I32, I32, T, P], I32),
        "vae_space_to_depth": ([T, I32, I32, I32, T, P], I32),
        "vae_tile_split": ([D, ctypes.POINTER(vae_tile_t), I32, ctypes.POINTER(I32)], I32),
        "vae_tile_merge": ([T, ctypes.POINTER(vae_tile_t), D, T, I32, P], I32),
        "vae_decoder_create": ([ctypes.POINTER(vae_decoder_spec_t), ctypes.POINTER(P), I32,
                                ctypes.POINTER(P)], I32),
        "vae_decoder_destroy": ([P], None),
        "vae_decoder_set_launch": ([P, I32], I32),
        "vae_decoder_set_clip_frames": ([P, I32], I32),
        "vae_decode_workspace_size": ([P, D, ctypes.POINTER(SZ)], I32),
        "vae_decode_tiled": ([P, T, D, T, P, SZ, P], I32),
        "vae_decode_status": ([P, D, P, SZ, ctypes.POINTER(I32), P], I32),
        "vae_decoder_set_timing": ([P, I32], I32),
        "vae_decoder_get_timing": ([P, ctypes.POINTER(vae_op_timing_t), I32,
                                    ctypes.POINTER(I32)], I32),
    }
    for name in EXPORTS:
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = sig[name]
    return lib


LIB = _load()


class VaeError(RuntimeError):
    def __init__(self, status, message, info):
        super().__init__(f"vae status {status}: {message}")
        self.status = status
        self.info = info


def _check(status):
    if status != VAE_OK:
        info = vae_error_info_t()
        LIB.vae_last_error_info(ctypes.byref(info))
        msg = LIB.vae_last_error().decode()
        raise VaeError(status, msg, {k: getattr(info, k) for k, _ in info._fields_})


def last_error_info():
    info = vae_error_info_t()
    LIB.vae_last_error_info(ctypes.byref(info))
    return {k: getattr(info, k) for k, _ in info._fields_}


# ------------------------------------------------------------------------------------------------
# Marshalling helpers
# ------------------------------------------------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return VAE_DTYPE_BF16
    if t.dtype == torch.float32:
        return VAE_DTYPE_F32
    if t.dtype == torch.float16:
        return VAE_DTYPE_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def tensor_desc(t):
    """vae_tensor_t of a contiguous NDHWC torch tensor (device memory)."""
    if t.dim() != 5:
        raise ValueError("expected an NDHWC tensor [N, T, H, W, C]")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous (NDHWC dense)")
    n, tt, h, w, c = t.shape
    return vae_tensor_t(t.data_ptr(), _dtype_code(t), 0, n, tt, h, w, c)


def box(b):
    if b is None:
        return None
    return vae_box_t(*[int(v) for v in b])


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ref(s):
    return None if s is None else ctypes.byref(s)


def _workspace(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------------------
# Entry points (names as in include/vae.h)
# ------------------------------------------------------------------------------------------------

def vae_conv3d_causal_strided(x, weight, bias, residual, y, stride, pad="around", out_box=None,
                              flags=0, weight_dtype=None, stream=None):
    """Strided causal Conv3d; weight is [Cout, 3, 3, 3, Cin] (bf16 or fp32), or a packed copy
    (uint8 buffer, with flags VAE_CONV_PACKED_WEIGHTS / VAE_CONV_PACKED_F16_WEIGHTS; its dtype is
    then bf16). pad: "around" or "after"."""
    xd, yd = tensor_desc(x), tensor_desc(y)
    rd = tensor_desc(residual) if residual is not None else None
    wdt = weight_dtype if weight_dtype is not None else (
        VAE_DTYPE_BF16 if flags else _dtype_code(weight))
    st, sh, sw = (int(s) for s in stride)
    _check(LIB.vae_conv3d_causal_strided(ctypes.byref(xd), _ptr(weight), wdt, _ptr(bias),
                                         _ref(rd), ctypes.byref(yd), _ref(box(out_box)), st, sh,
                                         sw, PAD_CODES[pad], int(flags), _stream(stream)))
    return y


def vae_conv3d_causal(x, weight, bias, residual, y, out_box=None, flags=0, stream=None):
    """Causal Conv3d; weight is a [Cout, 3, 3, 3, Cin] device tensor (bf16 or fp32)."""
    xd, yd = tensor_desc(x), tensor_desc(y)
    rd = tensor_desc(residual) if residual is not None else None
    _check(LIB.vae_conv3d_causal(ctypes.byref(xd), _ptr(weight), _dtype_code(weight), _ptr(bias),
                                 _ref(rd), ctypes.byref(yd), _ref(box(out_box)), int(flags),
                                 _stream(stream)))
    return y


def _fused_args(x, weight, bias, residual, y, out_box, flags, d2s, gn_groups, gn_eps,
                gn_mean_rstd, ws, in_up=(0, 0), in_scale_shift=None):
    keep = [tensor_desc(x), tensor_desc(y),
            tensor_desc(residual) if residual is not None else None, box(out_box)]
    a = vae_conv_fused_t()
    a.x = ctypes.pointer(keep[0])
    a.weight = _ptr(weight)
    a.weight_dtype = _dtype_code(weight)
    a.flags = int(flags)
    a.bias = _ptr(bias)
    a.residual = ctypes.pointer(keep[2]) if keep[2] is not None else None
    a.y = ctypes.pointer(keep[1])
    a.out_box = ctypes.pointer(keep[3]) if keep[3] is not None else None
    a.d2s_st, a.d2s_sh, a.d2s_sw = (int(f) for f in d2s)
    a.gn_groups = int(gn_groups)
    a.gn_eps = float(gn_eps)
    a.gn_mean_rstd = _ptr(gn_mean_rstd)
    a.ws = _ptr(ws)
    a.ws_bytes = ws.numel() if ws is not None else 0
    a.in_up_sh, a.in_up_sw = (int(f) for f in in_up)
    a.in_scale_shift = _ptr(in_scale_shift)
    return a, keep


def vae_conv3d_causal_fused_workspace(x, weight, y, out_box=None, d2s=(0, 0, 0), gn_groups=0,
                                      in_up=(0, 0), flags=0, in_scale_shift=None):
    a, keep = _fused_args(x, weight, None, None, y, out_box, flags, d2s, gn_groups, 0.0, None,
                          None, in_up, in_scale_shift)
    n = ctypes.c_size_t(0)
    _check(LIB.vae_conv3d_causal_fused_workspace(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def vae_conv3d_causal_fused(x, weight, bias, residual, y, out_box=None, flags=0, d2s=(0, 0, 0),
                            gn_groups=0, gn_eps=1e-6, gn_mean_rstd=None, ws=None, stream=None,
                            in_up=(0, 0), in_scale_shift=None):
    """Causal Conv3d of the nearest upsampling of x by in_up = (sh, sw), with a fused
    depth-to-space (d2s = (st, sh, sw), y is then the upsampled tensor) and/or the statistics of a
    GroupNorm over y (gn_mean_rstd [N, gn_groups, 2] fp32). With in_scale_shift ([N, Cin, 2]
    fp32, vae_groupnorm_scale_shift) the conv reads silu(x * scale + shift)."""
    if ws is None:
        n = vae_conv3d_causal_fused_workspace(x, weight, y, out_box, d2s, gn_groups, in_up, flags,
                                              in_scale_shift)
        ws = _workspace(n, x.device) if n else None
    a, keep = _fused_args(x, weight, bias, residual, y, out_box, flags, d2s, gn_groups, gn_eps,
                          gn_mean_rstd, ws, in_up, in_scale_shift)
    _check(LIB.vae_conv3d_causal_fused(ctypes.byref(a), _stream(stream)))
    return y


def vae_conv_weight_pack(weight, stream=None):
    """Fragment-packed copy of a bf16 [Cout, 3, 3, 3, Cin] device weight (a new uint8 tensor)."""
    return _pack(LIB.vae_conv_weight_pack, weight, stream)


def vae_conv_weight_pack_f16(weight, stream=None):
    """The same packed layout holding fp16(w * 2^10): the weights of an fp16-input conv."""
    return _pack(LIB.vae_conv_weight_pack_f16, weight, stream)


def _pack(fn, weight, stream):
    import torch
    cout, cin = weight.shape[0], weight.shape[-1]
    n = ctypes.c_size_t()
    _check(LIB.vae_conv_weight_pack_size(cout, cin, ctypes.byref(n)))
    packed = torch.empty(n.value, dtype=torch.uint8, device=weight.device)
    _check(fn(_ptr(weight), cout, cin, _ptr(packed), _stream(stream)))
    return packed


def _boxes(boxes):
    if boxes is None:
        return None, 1
    arr = (vae_box_t * len(boxes))(*[box(b) for b in boxes])
    return arr, len(boxes)


def vae_groupnorm_silu_workspace(x, boxes, groups):
    xd = tensor_desc(x)
    arr, nb = _boxes(boxes)
    n = ctypes.c_size_t()
    _check(LIB.vae_groupnorm_silu_workspace(ctypes.byref(xd), arr, nb, groups, ctypes.byref(n)))
    return n.value


def vae_groupnorm_silu_noalloc(x, boxes, groups, eps, gamma, beta, apply_silu, y, stream=None):
    """vae_groupnorm_silu on the library's own fixed scratch: allocates nothing."""
    xd, yd = tensor_desc(x), tensor_desc(y)
    arr, nb = _boxes(boxes)
    _check(LIB.vae_groupnorm_silu_noalloc(ctypes.byref(xd), arr, nb, groups, eps, _ptr(gamma),
                                          _ptr(beta), int(apply_silu), ctypes.byref(yd),
                                          _stream(stream)))
    return y


def vae_groupnorm_silu(x, boxes, groups, eps, gamma, beta, apply_silu, y, ws=None, stream=None):
    xd, yd = tensor_desc(x), tensor_desc(y)
    arr, nb = _boxes(boxes)
    if ws is None:
        ws = _workspace(vae_groupnorm_silu_workspace(x, boxes, groups), x.device)
    _check(LIB.vae_groupnorm_silu(ctypes.byref(xd), arr, nb, groups, eps, _ptr(gamma), _ptr(beta),
                                  int(apply_silu), ctypes.byref(yd), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return y


def vae_groupnorm_stats(x, boxes, groups, part, ws=None, stream=None):
    xd = tensor_desc(x)
    arr, nb = _boxes(boxes)
    if ws is None:
        n = ctypes.c_size_t()
        _check(LIB.vae_groupnorm_stats_workspace(ctypes.byref(xd), arr, nb, groups,
                                                 ctypes.byref(n)))
        ws = _workspace(n.value, x.device)
    _check(LIB.vae_groupnorm_stats(ctypes.byref(xd), arr, nb, groups, _ptr(part), _ptr(ws),
                                   ws.numel(), _stream(stream)))
    return part


def vae_groupnorm_combine(part, n_parts, n, groups, eps, mean_rstd, stream=None):
    _check(LIB.vae_groupnorm_combine(_ptr(part), n_parts, n, groups, eps, _ptr(mean_rstd),
                                     _stream(stream)))
    return mean_rstd


def vae_groupnorm_apply(x, out_box, groups, mean_rstd, gamma, beta, apply_silu, y, stream=None):
    xd, yd = tensor_desc(x), tensor_desc(y)
    _check(LIB.vae_groupnorm_apply(ctypes.byref(xd), _ref(box(out_box)), groups, _ptr(mean_rstd),
                                   _ptr(gamma), _ptr(beta), int(apply_silu), ctypes.byref(yd),
                                   _stream(stream)))
    return y


def vae_groupnorm_scale_shift(mean_rstd, channels, groups, gamma, beta, scale_shift,
                              stream=None):
    """scale_shift [N, channels, 2] fp32 of the normalise step for mean_rstd [N, groups, 2]."""
    _check(LIB.vae_groupnorm_scale_shift(_ptr(mean_rstd), int(mean_rstd.shape[0]), int(channels),
                                         int(groups), _ptr(gamma), _ptr(beta), _ptr(scale_shift),
                                         _stream(stream)))
    return scale_shift


def vae_rmsnorm_silu(x, eps, gamma, beta, apply_silu, y, stream=None):
    xd, yd = tensor_desc(x), tensor_desc(y)
    _check(LIB.vae_rmsnorm_silu(ctypes.byref(xd), eps, _ptr(gamma), _ptr(beta), int(apply_silu),
                                ctypes.byref(yd), _stream(stream)))
    return y


def vae_frame_attention_workspace(x):
    xd = tensor_desc(x)
    n = ctypes.c_size_t()
    _check(LIB.vae_frame_attention_workspace(ctypes.byref(xd), ctypes.byref(n)))
    return n.value


def vae_frame_attention(x, eps, gamma, beta, w_qkv, b_qkv, w_out, b_out, y, ws=None, stream=None):
    """Single-head attention over each frame's positions, plus x (w_qkv [3C, C], w_out [C, C]
    bf16 device tensors)."""
    if ws is None:
        ws = _workspace(vae_frame_attention_workspace(x), x.device)
    xd, yd = tensor_desc(x), tensor_desc(y)
    _check(LIB.vae_frame_attention(ctypes.byref(xd), eps, _ptr(gamma), _ptr(beta), _ptr(w_qkv),
                                   _ptr(b_qkv), _ptr(w_out), _ptr(b_out), ctypes.byref(yd),
                                   _ptr(ws), ws.numel(), _stream(stream)))
    return y


def vae_upsample(x, in_box, mode, st, sh, sw, y, stream=None):
    xd, yd = tensor_desc(x), tensor_desc(y)
    _check(LIB.vae_upsample(ctypes.byref(xd), _ref(box(in_box)), mode, st, sh, sw,
                            ctypes.byref(yd), _stream(stream)))
    return y


def vae_space_to_depth(x, st, sh, sw, y, stream=None):
    xd, yd = tensor_desc(x), tensor_desc(y)
    _check(LIB.vae_space_to_depth(ctypes.byref(xd), st, sh, sw, ctypes.byref(yd),
                                  _stream(stream)))
    return y


def tiling_desc(mode, latent_shape, scale, patches=(1, 1), tile=(0, 0), stride=(0, 0), tile_t=0,
                stride_t=0, down=(0, 0, 0)):
    """vae_tiling_desc_t from the NDHWC input shape [N, T, H, W, C] (a decoder's latent, an
    encoder's video). ``tile`` and ``stride`` are (H, W); ``tile_t`` > 0 also cuts T
    (overlap-blend only). ``down``: an encoder's folds (T, H, W); its tile grid is then cut on the
    output latent grid."""
    n, t, h, w = latent_shape[:4]
    return vae_tiling_desc_t(mode, n, t, h, w, scale[0], scale[1], scale[2], patches[0],
                             patches[1], tile[0], tile[1], stride[0], stride[1], tile_t, stride_t,
                             down[0], down[1], down[2])


def vae_tile_split(desc):
    """Host-only. Returns the list of vae_tile_t."""
    n = ctypes.c_int32()
    _check(LIB.vae_tile_split(ctypes.byref(desc), None, 0, ctypes.byref(n)))
    arr = (vae_tile_t * max(n.value, 1))()
    _check(LIB.vae_tile_split(ctypes.byref(desc), arr, n.value, ctypes.byref(n)))
    return list(arr[:n.value])


def vae_tile_merge(tile_out, tile, desc, out, flags, stream=None):
    td, od = tensor_desc(tile_out), tensor_desc(out)
    _check(LIB.vae_tile_merge(ctypes.byref(td), ctypes.byref(tile), ctypes.byref(desc),
                              ctypes.byref(od), flags, _stream(stream)))
    return out


_OPS = {"conv": VAE_OP_CONV, "res": VAE_OP_RES, "gn_silu": VAE_OP_GN_SILU, "d2s": VAE_OP_D2S,
        "nearest": VAE_OP_NEAREST, "res_rms": VAE_OP_RES_RMS, "rms_silu": VAE_OP_RMS_SILU,
        "attn": VAE_OP_ATTN, "s2d": VAE_OP_S2D}


def layer_descs(plan):
    out = []
    for op in plan:
        k = op["op"]
        if k == "conv":
            out.append(vae_layer_desc_t(VAE_OP_CONV, op["cin"], op["cout"], 1, 1, 1,
                                        int(op.get("f32_out", False)),
                                        int(op.get("no_split", False))))
        elif k == "res":
            out.append(vae_layer_desc_t(VAE_OP_RES, op["c"], op["c"], 1, 1, 1, 0, 0))
        elif k == "gn_silu":
            out.append(vae_layer_desc_t(VAE_OP_GN_SILU, 0, 0, 1, 1, 1, 0, 0))
        elif k == "res_rms":
            out.append(vae_layer_desc_t(VAE_OP_RES_RMS, op["c"], op["c"], 1, 1, 1, 0, 0))
        elif k == "rms_silu":
            out.append(vae_layer_desc_t(VAE_OP_RMS_SILU, 0, 0, 1, 1, 1, 0, 0))
        elif k == "attn":
            out.append(vae_layer_desc_t(VAE_OP_ATTN, op["c"], op["c"], 1, 1, 1, 0, 0))
        elif k == "s2d":
            out.append(vae_layer_desc_t(VAE_OP_S2D, 0, 0, op["st"], op["sh"], op["sw"], 0, 0))
        elif k == "d2s":
            out.append(vae_layer_desc_t(VAE_OP_D2S, 0, 0, op["st"], op["sh"], op["sw"], 0, 0))
        elif k == "nearest":
            out.append(vae_layer_desc_t(VAE_OP_NEAREST, 0, 0, 1, op["sh"], op["sw"], 0, 0))
        elif k == "conv_down":
            out.append(vae_layer_desc_t(VAE_OP_CONV_DOWN, op["cin"], op["cout"], op["st"],
                                        op["sh"], op["sw"], int(op.get("f32_out", False)), 0,
                                        PAD_CODES[op["pad"]]))
        else:
            raise ValueError(k)
    return out


class Decoder:
    """vae_decoder_t over a layer plan and device parameter tensors (plan order, two per entry).

    ``params`` is a flat list of device tensors or None: conv -> (weight [Cout,3,3,3,Cin], bias),
    GN / RMS -> (gamma, beta), attn -> (gamma, beta, w_qkv, b_qkv, w_out, b_out); the tensors must
    outlive the decoder.
    """

    def __init__(self, dtype, latent_channels, groups, eps, plan, params, act_dtype=VAE_DTYPE_F32,
                 flags=0):
        self._keep = list(params)
        descs = layer_descs(plan)
        self._layers = (vae_layer_desc_t * len(descs))(*descs)
        spec = vae_decoder_spec_t(dtype, act_dtype, flags, latent_channels, groups, eps, len(descs),
                                  self._layers)
        ptrs = (ctypes.c_void_p * max(len(params), 1))(
            *[None if p is None else p.data_ptr() for p in params])
        h = ctypes.c_void_p()
        _check(LIB.vae_decoder_create(ctypes.byref(spec), ptrs, len(params), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            LIB.vae_decoder_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def pack_weights(self, device, stream=None):
        """Allocate the packed-weight buffer (kept alive by the decoder) and pack into it."""
        import torch
        n = ctypes.c_size_t()
        _check(LIB.vae_decoder_packed_weight_size(self._h, ctypes.byref(n)))
        self._packed = torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)
        _check(LIB.vae_decoder_pack_weights(self._h, _ptr(self._packed), self._packed.numel(),
                                            _stream(stream)))

    def set_launch(self, launch):
        """VAE_LAUNCH_MERGED or VAE_LAUNCH_PER_PATCH (patch-halo decodes); query the workspace
        size afterwards."""
        _check(LIB.vae_decoder_set_launch(self._h, int(launch)))

    def set_clip_frames(self, frames):
        """Decode patch-halo tilings clip by clip, `frames` latent frames at a time, carrying each
        causal conv's last two input frames (0: all frames at once); query the workspace size
        afterwards."""
        _check(LIB.vae_decoder_set_clip_frames(self._h, int(frames)))

    def workspace_size(self, desc):
        n = ctypes.c_size_t()
        _check(LIB.vae_decode_workspace_size(self._h, ctypes.byref(desc), ctypes.byref(n)))
        return n.value

    def vae_decode_tiled(self, latent, desc, out, ws, stream=None):
        ld, od = tensor_desc(latent), tensor_desc(out)
        _check(LIB.vae_decode_tiled(self._h, ctypes.byref(ld), ctypes.byref(desc),
                                    ctypes.byref(od), _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def status(self, desc, ws, stream=None):
        """Flags of the last decode through `ws` (VAE_STATUS_NONFINITE); synchronises."""
        f = ctypes.c_int32()
        _check(LIB.vae_decode_status(self._h, ctypes.byref(desc), _ptr(ws), ws.numel(),
                                     ctypes.byref(f), _stream(stream)))
        return f.value

    def set_timing(self, enable):
        _check(LIB.vae_decoder_set_timing(self._h, int(enable)))

    def timing(self):
        n = ctypes.c_int32()
        _check(LIB.vae_decoder_get_timing(self._h, None, 0, ctypes.byref(n)))
        arr = (vae_op_timing_t * max(n.value, 1))()
        _check(LIB.vae_decoder_get_timing(self._h, arr, n.value, ctypes.byref(n)))
        return [{"kind": VAE_KIND_NAMES[r.kind], "layer": r.layer, "tile": r.tile, "ms": r.ms,
                 "flops": r.flops, "bytes": r.bytes} for r in arr[:n.value]]
