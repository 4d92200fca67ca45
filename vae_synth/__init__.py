"""Seeded synthetic inputs and workload descriptions for the tiled causal 3-D VAE decode.

This module is shared by the CPU oracle and the GPU path and holds none of the method's arithmetic:
- the layer plan of each decoder workload (shapes only);
- random draws from numpy's PCG64 with fixed seeds;
- the rounding of drawn values to bfloat16 (round-to-nearest-even), so that both sides receive the
  very same numbers.

Workloads (the pages publish no checkpoints, so every weight is random-init, as the DistVAE PR #14
"Add tiled VAE parallelism & extended model support" does in its benchmark harness commit, where a VAE
is built from its config.json with random weights):
- ``CONV_GN``: one causal Conv3d 32->32 followed by GroupNorm(8)+SiLU on [1,32,5,32,32], fp32.
- ``TINY_DECODER``: a small fp32 causal decoder, latent [1,16,3,16,16] -> video [1,3,5,64,64].
- ``LTX2_720P``: an LTX-2-shaped bf16 decoder, latent [1,128,16,22,40] -> video [1,3,121,704,1280].
- ``LTX2_SMALL`` / ``LTX2_MID``: the same layer plan at small latents, for parity at oracle-friendly
  sizes;
- ``LTX2_720P_1F``: the same plan on one latent frame at the full 720p extent [1,128,1,22,40];
- ``LTX2_TINY``: the same structure at a quarter of the widths, for a quick smoke check;
  ``LTX2_TINY_N2`` is that plan on a batch of two latents.
- ``WAN_720P``: a Wan2.2-TI2V-5B-shaped bf16 decoder, latent [1,48,21,44,80] -> video
  [1,3,81,704,1280]: RMS-norm residual blocks, a mid-block single-head frame attention, two
  temporal and three spatial (nearest + conv) upsamplings, unpatchify 2x2. ``WAN_SMALL`` and
  ``WAN_TINY`` are that plan at oracle-friendly sizes (full and quarter widths).

Layer plan vocabulary (every op works on a channels-last activation):
- ``conv``: causal Conv3d 3x3x3, stride 1, ``cin`` -> ``cout``; ``"f32_out": True`` keeps the result
  in fp32 (the last convolution of a bf16 decoder). ``"no_split": True`` is a precision hint for the
  GPU path only (it has no effect on what is computed): that conv rounds an fp32 input to bf16 once
  instead of applying it as hi + lo bf16 operands. The LTX-2-shaped plan sets it on its largest
  upsampling conv, which saves a tenth of the decode time at 720p and keeps the decode within
  2e-2 max-abs of the oracle;
- ``res``: residual block of width ``c``: GN+SiLU, conv, GN+SiLU, conv, plus the block input;
- ``gn_silu``: GroupNorm followed by SiLU;
- ``res_rms`` / ``rms_silu``: the same with per-position RMS norms over the channels;
- ``attn``: single-head self-attention over each frame's positions, width ``c``, with its residual;
- ``d2s``: depth-to-space by (st, sh, sw); with st > 1 the first st-1 output frames are dropped;
- ``nearest``: nearest-neighbour spatial upsampling by (sh, sw).
- ``conv_down``: strided causal Conv3d 3x3x3, ``cin`` -> ``cout``, strides (st, sh, sw), zero
  padding ``pad`` = "around" (one row/column on every side) or "after" (one after the image
  only); T frames become (T - 1) // st + 1.

Parameters are drawn in plan order: each ``conv`` gives one weight [cout, cin, 3, 3, 3] and one bias
[cout]; each ``res`` / ``res_rms`` gives norm(c), conv(c, c), norm(c), conv(c, c); each ``gn_silu`` /
``rms_silu`` gives norm(c); each ``attn`` gives one dict with the norm's gamma/beta, w_qkv [3c, c],
b_qkv [3c], w_out [c, c], b_out [c]. Conv weight number k (0-based, counting every conv in plan
order) is N(0, 1) * 1/sqrt(27 * cin) drawn from PCG64([1, k]); attention block number k draws
w_qkv and w_out as N(0, 1) * 1/sqrt(c) from PCG64([5, k, 0]) and PCG64([5, k, 1]). Biases are 0,
norm gamma is 1 and beta is 0, unless ``affine_seed`` asks for random values (used by tests to
exercise the bias, gamma and beta paths).
"""
from __future__ import annotations

import copy

import numpy as np

__all__ = [
    "CONV_GN", "TINY_DECODER", "LTX2_720P", "LTX2_SMALL", "LTX2_MID", "LTX2_720P_1F", "LTX2_TINY",
    "LTX2_TINY_N2", "WAN_720P", "WAN_SMALL", "WAN_720P_1F", "WAN_720P_6F", "WAN_TINY",
    "MIXED_RMS_GN", "WORKLOADS",
    "round_bf16", "bf16_bits", "normal", "uniform", "latent", "decoder_params", "conv_params",
    "walk_plan", "with_latent",
]


# ----------------------------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------------------------

CONV_GN = {
    "name": "conv_gn_32",
    "dtype": "f32",
    "input": (1, 32, 5, 32, 32),          # N, C, T, H, W
    "cin": 32, "cout": 32, "groups": 8, "eps": 1e-6,
    "patches_w": 2,
}

TINY_DECODER = {
    "name": "tiny_decoder",
    "dtype": "f32",
    "latent": (1, 16, 3, 16, 16),
    "groups": 32, "eps": 1e-6,
    "layers": [
        {"op": "conv", "cin": 16, "cout": 128},
        {"op": "res", "c": 128},
        {"op": "res", "c": 128},
        {"op": "res", "c": 128},
        {"op": "nearest", "sh": 2, "sw": 2},
        {"op": "conv", "cin": 128, "cout": 64},
        {"op": "res", "c": 64},
        {"op": "nearest", "sh": 2, "sw": 2},
        {"op": "conv", "cin": 64, "cout": 32},
        {"op": "conv", "cin": 32, "cout": 64},
        {"op": "d2s", "st": 2, "sh": 1, "sw": 1},
        {"op": "gn_silu"},
        {"op": "conv", "cin": 32, "cout": 3},
    ],
    "scale": (2, 4, 4),                   # latent -> video: T_out = 1 + (T-1)*2, H*4, W*4
    "patch_grid": (2, 2),
    "overlap_tile": (8, 8), "overlap_stride": (6, 6),
}

_LTX2_LAYERS = [
    {"op": "conv", "cin": 128, "cout": 1024},
    {"op": "res", "c": 1024},
    {"op": "res", "c": 1024},
    {"op": "conv", "cin": 1024, "cout": 4096},
    {"op": "d2s", "st": 2, "sh": 2, "sw": 2},
    {"op": "res", "c": 512},
    {"op": "res", "c": 512},
    {"op": "conv", "cin": 512, "cout": 2048},
    {"op": "d2s", "st": 2, "sh": 2, "sw": 2},
    {"op": "res", "c": 256},
    {"op": "res", "c": 256},
    # the largest upsampling conv rounds its fp32 input to bf16 once (see the module docstring)
    {"op": "conv", "cin": 256, "cout": 1024, "no_split": True},
    {"op": "d2s", "st": 2, "sh": 2, "sw": 2},
    {"op": "res", "c": 128},
    {"op": "res", "c": 128},
    {"op": "gn_silu"},
    {"op": "conv", "cin": 128, "cout": 48, "f32_out": True},
    {"op": "d2s", "st": 1, "sh": 4, "sw": 4},
]

LTX2_720P = {
    "name": "ltx2_720p",
    "dtype": "bf16",
    "latent": (1, 128, 16, 22, 40),
    "groups": 32, "eps": 1e-6,
    "layers": _LTX2_LAYERS,
    "scale": (8, 32, 32),
    "patch_grid": (1, 4),
    "overlap_tile": (16, 16), "overlap_stride": (14, 14),
}


def with_latent(spec: dict, latent_shape, name: str, **extra) -> dict:
    """A copy of ``spec`` with another latent shape (and optionally other tiling fields)."""
    out = copy.deepcopy(spec)
    out["latent"] = tuple(latent_shape)
    out["name"] = name
    out.update(extra)
    return out


LTX2_SMALL = with_latent(LTX2_720P, (1, 128, 2, 3, 5), "ltx2_small",
                         patch_grid=(1, 2), overlap_tile=(3, 4), overlap_stride=(2, 3))
LTX2_MID = with_latent(LTX2_720P, (1, 128, 3, 4, 6), "ltx2_mid",
                       patch_grid=(2, 3), overlap_tile=(3, 4), overlap_stride=(2, 3))
# One latent frame at the full 720p extent: every output value of the full-width plan can be
# compared with the oracle in seconds.
LTX2_720P_1F = with_latent(LTX2_720P, (1, 128, 1, 22, 40), "ltx2_720p_1f")

# The LTX-2 layer plan at a quarter of the widths (256/128/64/32), on a small latent: every kernel
# path of the 720p plan at a size the oracle decodes in about a second (smoke check).
LTX2_TINY = {
    "name": "ltx2_tiny",
    "dtype": "bf16",
    "latent": (1, 128, 2, 4, 6),
    "groups": 32, "eps": 1e-6,
    "layers": [
        {"op": "conv", "cin": 128, "cout": 256},
        {"op": "res", "c": 256},
        {"op": "conv", "cin": 256, "cout": 1024},
        {"op": "d2s", "st": 2, "sh": 2, "sw": 2},
        {"op": "res", "c": 128},
        {"op": "conv", "cin": 128, "cout": 512},
        {"op": "d2s", "st": 2, "sh": 2, "sw": 2},
        {"op": "res", "c": 64},
        {"op": "conv", "cin": 64, "cout": 256},
        {"op": "d2s", "st": 2, "sh": 2, "sw": 2},
        {"op": "res", "c": 32},
        {"op": "gn_silu"},
        {"op": "conv", "cin": 32, "cout": 48, "f32_out": True},
        {"op": "d2s", "st": 1, "sh": 4, "sw": 4},
    ],
    "scale": (8, 32, 32),
    "patch_grid": (1, 2),
    "overlap_tile": (3, 4), "overlap_stride": (2, 3),
}

# Two samples in one latent: every per-sample path (GroupNorm statistics, tile offsets) at N = 2.
LTX2_TINY_N2 = with_latent(LTX2_TINY, (2, 128, 2, 4, 6), "ltx2_tiny_n2")

_WAN_LAYERS = [
    {"op": "conv", "cin": 48, "cout": 1024},
    {"op": "res_rms", "c": 1024},                                   # mid block
    {"op": "attn", "c": 1024},
    {"op": "res_rms", "c": 1024},
    {"op": "res_rms", "c": 1024},                                   # stage 0
    {"op": "conv", "cin": 1024, "cout": 2048},                       # temporal x2
    {"op": "d2s", "st": 2, "sh": 1, "sw": 1},
    {"op": "nearest", "sh": 2, "sw": 2},                            # spatial x2
    {"op": "conv", "cin": 1024, "cout": 512},
    {"op": "res_rms", "c": 512},                                    # stage 1
    {"op": "conv", "cin": 512, "cout": 1024},                        # temporal x2
    {"op": "d2s", "st": 2, "sh": 1, "sw": 1},
    {"op": "nearest", "sh": 2, "sw": 2},                            # spatial x2
    {"op": "conv", "cin": 512, "cout": 256},
    {"op": "res_rms", "c": 256},                                    # stage 2
    {"op": "nearest", "sh": 2, "sw": 2},                            # spatial x2
    {"op": "conv", "cin": 256, "cout": 128},
    {"op": "res_rms", "c": 128},                                    # stage 3
    {"op": "rms_silu"},
    {"op": "conv", "cin": 128, "cout": 12, "f32_out": True},
    {"op": "d2s", "st": 1, "sh": 2, "sw": 2},                       # unpatchify 2x2
]

WAN_720P = {
    "name": "wan_720p",
    "dtype": "bf16",
    "latent": (1, 48, 21, 44, 80),
    "groups": 32, "eps": 1e-6,
    "layers": _WAN_LAYERS,
    "scale": (4, 16, 16),
    "patch_grid": (1, 4),
    "overlap_tile": (32, 32), "overlap_stride": (28, 28),
}
WAN_SMALL = with_latent(WAN_720P, (1, 48, 2, 3, 5), "wan_small",
                        patch_grid=(1, 2), overlap_tile=(2, 4), overlap_stride=(1, 3))
# One latent frame at the full 720p extent: the attention sees all 44 x 80 positions of the frame.
WAN_720P_1F = with_latent(WAN_720P, (1, 48, 1, 44, 80), "wan_720p_1f")
# Six latent frames at the full 720p extent (21 output frames): both temporal upsamplings and the
# causal temporal taps at full spatial size, at a quarter of the full decode's work (the reference
# for its golden samples).
WAN_720P_6F = with_latent(WAN_720P, (1, 48, 6, 44, 80), "wan_720p_6f")

# The Wan plan at a quarter of the widths (256/128/64/32).
WAN_TINY = with_latent(WAN_720P, (1, 48, 3, 4, 6), "wan_tiny",
                       patch_grid=(2, 2), overlap_tile=(3, 4), overlap_stride=(2, 3))
WAN_TINY["layers"] = [dict(op) for op in _WAN_LAYERS]
for _op in WAN_TINY["layers"]:
    for _k in ("cin", "cout", "c"):
        if _k in _op and not (_k == "cin" and _op["cin"] == 48) and \
                not (_k == "cout" and _op.get("f32_out")):
            _op[_k] //= 4

# The Wan-shaped decoder is described with both RMS-style norms and GroupNorm variants: an RMS
# residual block whose output feeds a GroupNorm (its second conv then gathers the GroupNorm's
# statistics), at a size the oracle decodes in a second.
MIXED_RMS_GN = {
    "name": "mixed_rms_gn",
    "dtype": "bf16",
    "latent": (1, 32, 3, 12, 20),
    "groups": 32, "eps": 1e-6,
    "layers": [
        {"op": "conv", "cin": 32, "cout": 128},
        {"op": "res_rms", "c": 128},
        {"op": "gn_silu"},
        {"op": "conv", "cin": 128, "cout": 32, "f32_out": True},
    ],
    "scale": (1, 1, 1),
    "patch_grid": (1, 2),
    "overlap_tile": (6, 8), "overlap_stride": (4, 6),
}

# LTX-2-shaped encoder: video [1,3,121,704,1280] -> latent [1,256,16,22,40] (mean and log-variance,
# 128 channels each), widths 128/256/512/1024. Each downsampler is a stride-1 causal conv to
# C_next / 8 channels, then a (2,2,2) space-to-depth fold with the causal front pad (121 -> 61 -> 31
# -> 16 frames); the input is patchified by a (1,4,4) fold first.
_LTX2_ENC_LAYERS = [
    {"op": "s2d", "st": 1, "sh": 4, "sw": 4},                       # patchify: 3 -> 48 channels
    {"op": "conv", "cin": 48, "cout": 128},
    {"op": "res", "c": 128},
    {"op": "res", "c": 128},
    {"op": "conv", "cin": 128, "cout": 32},
    {"op": "s2d", "st": 2, "sh": 2, "sw": 2},
    {"op": "res", "c": 256},
    {"op": "res", "c": 256},
    {"op": "conv", "cin": 256, "cout": 64},
    {"op": "s2d", "st": 2, "sh": 2, "sw": 2},
    {"op": "res", "c": 512},
    {"op": "res", "c": 512},
    {"op": "conv", "cin": 512, "cout": 128},
    {"op": "s2d", "st": 2, "sh": 2, "sw": 2},
    {"op": "res", "c": 1024},
    {"op": "res", "c": 1024},
    {"op": "gn_silu"},
    {"op": "conv", "cin": 1024, "cout": 256, "f32_out": True},
]

LTX2_ENC_720P = {
    "name": "ltx2_enc_720p",
    "kind": "encoder",
    "dtype": "bf16",
    "input": (1, 3, 121, 704, 1280),
    "groups": 32, "eps": 1e-6,
    "layers": _LTX2_ENC_LAYERS,
    "down": (8, 32, 32),                  # video -> latent: T = (T_in + 7) / 8, H / 32, W / 32
    "patch_grid": (1, 4),
    # tiles on the latent grid: 16 / 14 latent rows are 512 / 448 pixels (64 pixels of overlap)
    "overlap_tile": (16, 16), "overlap_stride": (14, 14),
}


def with_input(spec: dict, input_shape, name: str, **extra) -> dict:
    """A copy of an encoder ``spec`` with another input shape (and other tiling fields)."""
    out = copy.deepcopy(spec)
    out["input"] = tuple(input_shape)
    out["name"] = name
    out.update(extra)
    return out


LTX2_ENC_TINY = with_input(LTX2_ENC_720P, (1, 3, 9, 64, 96), "ltx2_enc_tiny", patch_grid=(1, 3),
                           overlap_tile=(2, 2), overlap_stride=(1, 1))
LTX2_ENC_SMALL = with_input(LTX2_ENC_720P, (1, 3, 9, 64, 160), "ltx2_enc_small",
                            patch_grid=(2, 2), overlap_tile=(2, 3), overlap_stride=(2, 2))

# The same encoder with bare strided downsamplers: each downsampler is one causal Conv3d C ->
# C_next with stride (2, 2, 2) (LTX-2's fourth downsample kind), zero padding one row and column
# around; the frame counts follow the causal rule (T - 1) // 2 + 1: 121 -> 61 -> 31 -> 16.
_LTX2_ENC_STRIDED_LAYERS = [
    {"op": "s2d", "st": 1, "sh": 4, "sw": 4},
    {"op": "conv", "cin": 48, "cout": 128},
    {"op": "res", "c": 128},
    {"op": "res", "c": 128},
    {"op": "conv_down", "cin": 128, "cout": 256, "st": 2, "sh": 2, "sw": 2, "pad": "around"},
    {"op": "res", "c": 256},
    {"op": "res", "c": 256},
    {"op": "conv_down", "cin": 256, "cout": 512, "st": 2, "sh": 2, "sw": 2, "pad": "around"},
    {"op": "res", "c": 512},
    {"op": "res", "c": 512},
    {"op": "conv_down", "cin": 512, "cout": 1024, "st": 2, "sh": 2, "sw": 2, "pad": "around"},
    {"op": "res", "c": 1024},
    {"op": "res", "c": 1024},
    {"op": "gn_silu"},
    {"op": "conv", "cin": 1024, "cout": 256, "f32_out": True},
]
LTX2_ENC_STRIDED_720P = with_input(LTX2_ENC_720P, LTX2_ENC_720P["input"], "ltx2_enc_strided_720p")
LTX2_ENC_STRIDED_720P["layers"] = _LTX2_ENC_STRIDED_LAYERS
LTX2_ENC_STRIDED_TINY = with_input(LTX2_ENC_STRIDED_720P, (1, 3, 9, 64, 96),
                                   "ltx2_enc_strided_tiny", patch_grid=(1, 3),
                                   overlap_tile=(2, 2), overlap_stride=(1, 1))
# A Wan-style downsampler: zero padding only after the image (0, 1, 0, 1), then stride 2 in space
# (and 1 in time), at a quarter of the widths.
WAN_ENC_TINY = {
    "name": "wan_enc_tiny",
    "kind": "encoder",
    "dtype": "bf16",
    "input": (1, 3, 5, 32, 48),
    "groups": 32, "eps": 1e-6,
    "layers": [
        {"op": "s2d", "st": 1, "sh": 2, "sw": 2},
        {"op": "conv", "cin": 12, "cout": 64},
        {"op": "res_rms", "c": 64},
        {"op": "conv_down", "cin": 64, "cout": 128, "st": 1, "sh": 2, "sw": 2, "pad": "after"},
        {"op": "res_rms", "c": 128},
        {"op": "conv_down", "cin": 128, "cout": 128, "st": 2, "sh": 2, "sw": 2, "pad": "after"},
        {"op": "res", "c": 128},
        {"op": "gn_silu"},
        {"op": "conv", "cin": 128, "cout": 32, "f32_out": True},
    ],
    "down": (2, 8, 8),
    "patch_grid": (2, 2),
    "overlap_tile": (3, 3), "overlap_stride": (2, 2),
}

WORKLOADS = {s["name"]: s for s in (CONV_GN, TINY_DECODER, LTX2_720P, LTX2_SMALL, LTX2_MID,
                                    LTX2_720P_1F, LTX2_TINY, LTX2_TINY_N2, WAN_720P, WAN_SMALL,
                                    WAN_720P_1F, WAN_720P_6F, WAN_TINY, MIXED_RMS_GN,
                                    LTX2_ENC_720P, LTX2_ENC_TINY, LTX2_ENC_SMALL,
                                    LTX2_ENC_STRIDED_720P, LTX2_ENC_STRIDED_TINY, WAN_ENC_TINY)}


# ----------------------------------------------------------------------------------------------
# Draws and bf16 rounding
# ----------------------------------------------------------------------------------------------

def bf16_bits(a) -> np.ndarray:
    """uint16 bit patterns of ``a`` rounded to bfloat16, round-to-nearest-even (finite inputs)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32)
    # finite inputs stay below 2^32 after adding the rounding bias, so uint32 does not wrap
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def round_bf16(a) -> np.ndarray:
    """``a`` rounded to the nearest bfloat16 (ties to even), returned as float32."""
    bits = bf16_bits(a).astype(np.uint32) << 16
    return bits.view(np.float32)


def normal(shape, seed, scale: float = 1.0, mean: float = 0.0, dtype: str = "f32") -> np.ndarray:
    """N(mean, scale^2) float32 draw from PCG64(seed); bf16-rounded when dtype == 'bf16'."""
    g = np.random.Generator(np.random.PCG64(seed))
    v = (g.standard_normal(size=tuple(shape)) * scale + mean).astype(np.float32)
    return round_bf16(v) if dtype == "bf16" else v


def uniform(shape, seed, lo: float = -1.0, hi: float = 1.0, dtype: str = "f32") -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    v = g.uniform(lo, hi, size=tuple(shape)).astype(np.float32)
    return round_bf16(v) if dtype == "bf16" else v


def latent(spec: dict, seed=0) -> np.ndarray:
    """The plan's input, NCDHW float32 (bf16-exact for bf16 workloads): a N(0, 1) latent for a
    decoder, a U(-1, 1) video for an encoder."""
    if spec.get("kind") == "encoder":
        return uniform(spec["input"], seed, dtype=spec["dtype"])
    shape = spec["latent"] if "latent" in spec else spec["input"]
    return normal(shape, seed, dtype=spec["dtype"])


def conv_params(index: int, cin: int, cout: int, dtype: str, affine_seed=None) -> dict:
    w = normal((cout, cin, 3, 3, 3), [1, index], scale=1.0 / np.sqrt(27.0 * cin), dtype=dtype)
    if affine_seed is None:
        b = np.zeros(cout, np.float32)
    else:
        b = normal((cout,), [2, affine_seed, index], scale=0.1)
    return {"kind": "conv", "w": w, "b": b, "cin": cin, "cout": cout}


def gn_params(index: int, c: int, affine_seed=None) -> dict:
    if affine_seed is None:
        gamma, beta = np.ones(c, np.float32), np.zeros(c, np.float32)
    else:
        gamma = normal((c,), [3, affine_seed, index], scale=0.2, mean=1.0)
        beta = normal((c,), [4, affine_seed, index], scale=0.1)
    return {"kind": "gn", "gamma": gamma, "beta": beta, "c": c}


def attn_params(index: int, c: int, dtype: str, affine_seed=None) -> dict:
    g = gn_params(1000 + index, c, affine_seed)
    w_qkv = normal((3 * c, c), [5, index, 0], scale=1.0 / np.sqrt(c), dtype=dtype)
    w_out = normal((c, c), [5, index, 1], scale=1.0 / np.sqrt(c), dtype=dtype)
    if affine_seed is None:
        b_qkv, b_out = np.zeros(3 * c, np.float32), np.zeros(c, np.float32)
    else:
        b_qkv = normal((3 * c,), [6, affine_seed, index, 0], scale=0.1)
        b_out = normal((c,), [6, affine_seed, index, 1], scale=0.1)
    return {"kind": "attn", "gamma": g["gamma"], "beta": g["beta"], "w_qkv": w_qkv,
            "b_qkv": b_qkv, "w_out": w_out, "b_out": b_out, "c": c}


def walk_plan(spec: dict):
    """Yield (op, channels_in, channels_out) along the plan, following the channel count only."""
    c = (spec["latent"] if "latent" in spec else spec["input"])[1]
    for op in spec["layers"]:
        kind = op["op"]
        if kind == "conv":
            yield op, op["cin"], op["cout"]
            c = op["cout"]
        elif kind in ("res", "res_rms", "attn"):
            yield op, op["c"], op["c"]
        elif kind in ("gn_silu", "rms_silu"):
            yield op, c, c
        elif kind == "d2s":
            k = op["st"] * op["sh"] * op["sw"]
            yield op, c, c // k
            c //= k
        elif kind == "nearest":
            yield op, c, c
        elif kind == "s2d":
            k = op["st"] * op["sh"] * op["sw"]
            yield op, c, c * k
            c *= k
        elif kind == "conv_down":
            yield op, op["cin"], op["cout"]
            c = op["cout"]
        else:
            raise ValueError(f"unknown op {kind!r}")


def decoder_params(spec: dict, affine_seed=None) -> list:
    """Parameter list of a decoder plan, in plan order (see the module docstring)."""
    out, n_conv, n_gn, n_attn = [], 0, 0, 0
    dt = spec["dtype"]
    for op, cin, cout in walk_plan(spec):
        kind = op["op"]
        if kind in ("conv", "conv_down"):
            out.append(conv_params(n_conv, cin, cout, dt, affine_seed)); n_conv += 1
        elif kind == "attn":
            out.append(attn_params(n_attn, cin, dt, affine_seed)); n_attn += 1
        elif kind in ("res", "res_rms"):
            out.append(gn_params(n_gn, cin, affine_seed)); n_gn += 1
            out.append(conv_params(n_conv, cin, cin, dt, affine_seed)); n_conv += 1
            out.append(gn_params(n_gn, cin, affine_seed)); n_gn += 1
            out.append(conv_params(n_conv, cin, cin, dt, affine_seed)); n_conv += 1
        elif kind in ("gn_silu", "rms_silu"):
            out.append(gn_params(n_gn, cin, affine_seed)); n_gn += 1
    return out
