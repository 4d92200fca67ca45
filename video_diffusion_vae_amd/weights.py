"""Upload a decoder's parameters to the device in the library's layouts.

This is setup-time marshalling, not part of the decode itself:
- conv weights go from [Cout, Cin, 3, 3, 3] to [Cout, 3, 3, 3, Cin] (the K dimension, taps then
  channels, contiguous per output channel);
- biases, gamma and beta become fp32 vectors.
"""
from __future__ import annotations

import numpy as np

from ._binding import (Decoder, VAE_DTYPE_BF16, VAE_DTYPE_F32, VAE_DECODE_F16_OPERANDS,
                       VAE_DECODE_NORM_IN_CONV, VAE_DECODE_SPLIT_FP32_OPERANDS)

# How convs that read an fp32 activation (the upsampling convs, conv_out) get their operands:
# "f16" (one rounding to fp16, bf16 rate), "split" (bf16 hi + lo, twice the work) or "bf16".
OPERAND_FLAGS = {"f16": VAE_DECODE_F16_OPERANDS, "split": VAE_DECODE_SPLIT_FP32_OPERANDS,
                 "bf16": 0}


def conv_weight_layout(w, dtype, device):
    """[Cout, Cin, 3, 3, 3] array -> contiguous device tensor [Cout, 3, 3, 3, Cin]."""
    import torch
    t = torch.as_tensor(np.ascontiguousarray(np.asarray(w, dtype=np.float32)))
    t = t.permute(0, 2, 3, 4, 1).contiguous()
    return t.to(device=device, dtype=dtype)


def _lead_fold(spec: dict) -> int:
    """Channel factor of the space-to-depth folds before the first conv (an encoder's patchify)."""
    k = 1
    for op in spec["layers"]:
        if op["op"] != "s2d":
            break
        k *= op["st"] * op["sh"] * op["sw"]
    return k


def latent_channels(spec: dict) -> int:
    """Channels of the input the GPU plan takes: the plan's, padded for a bf16 plan so that the
    first conv reads a multiple of 32 channels and runs on the matrix cores (a 48-channel latent
    -> 64; a 3-channel video -> 4, which the 4x4 patchify turns into 64). The extra channels are
    zeros in the input and in the first conv's weights, so the result is the same sum."""
    c = (spec["latent"] if "latent" in spec else spec["input"])[1]
    if spec["dtype"] != "bf16":
        return c
    k = _lead_fold(spec)
    while (c * k) % 32:
        c += 1
    return c


def pad_latent(z, spec: dict):
    """NDHWC host latent padded with zero channels to latent_channels(spec)."""
    c = latent_channels(spec)
    if z.shape[-1] == c:
        return z
    pad = np.zeros(z.shape[:-1] + (c - z.shape[-1],), dtype=z.dtype)
    return np.concatenate([z, pad], axis=-1)


def upload_decoder(spec: dict, params: list, device="cuda", act_dtype="f32", operands="f16",
                   packed=True, norm_in_conv=False):
    """Build a Decoder for a layer plan ``spec`` with parameter dicts in plan order.

    Each parameter dict is {"kind": "conv", "w", "b"} or {"kind": "gn", "gamma", "beta"} holding
    host arrays. ``act_dtype`` is the storage dtype of the activations between ops; the library
    takes "f32" only (it refuses bf16 storage, which misses the bf16 decode's accuracy bound).
    ``operands`` picks how convs that read an fp32 activation get their operands (OPERAND_FLAGS;
    bf16 plans only). ``packed`` gives the MFMA convs fragment-packed weight
    copies. ``norm_in_conv``: those convs apply the GroupNorm + SiLU of their input while staging
    it, instead of a normalise pass of its own (VAE_DECODE_NORM_IN_CONV). Returns the Decoder; it
    keeps the device tensors alive.
    """
    import torch
    tdt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
    f32 = lambda a: torch.as_tensor(np.asarray(a, np.float32)).to(device)
    lc = latent_channels(spec)
    c0 = (spec["latent"] if "latent" in spec else spec["input"])[1]
    fold = _lead_fold(spec)
    layers = [dict(op) for op in spec["layers"]]
    first_conv = next(i for i, op in enumerate(layers) if op["op"] == "conv")
    flat = []
    for k, p in enumerate(params):
        if p["kind"] == "conv":
            w = np.asarray(p["w"], np.float32)
            if k == 0 and lc > c0:
                # zero weights for the zero input channels: input channel f * c0 + j of the
                # (folded) plan input is channel f * lc + j of the padded one
                cout = w.shape[0]
                wp = np.zeros((cout, fold, lc) + w.shape[2:], np.float32)
                wp[:, :, :c0] = w.reshape((cout, fold, c0) + w.shape[2:])
                w = wp.reshape((cout, fold * lc) + w.shape[2:])
                layers[first_conv]["cin"] = fold * lc
            flat.append(conv_weight_layout(w, tdt, device))
            flat.append(f32(p["b"]))
        elif p["kind"] == "attn":
            flat += [f32(p["gamma"]), f32(p["beta"]),
                     torch.as_tensor(np.asarray(p["w_qkv"], np.float32)).to(device, tdt),
                     f32(p["b_qkv"]),
                     torch.as_tensor(np.asarray(p["w_out"], np.float32)).to(device, tdt),
                     f32(p["b_out"])]
        else:
            flat.append(f32(p["gamma"]))
            flat.append(f32(p["beta"]))
    code = VAE_DTYPE_BF16 if spec["dtype"] == "bf16" else VAE_DTYPE_F32
    act = VAE_DTYPE_BF16 if act_dtype == "bf16" else VAE_DTYPE_F32
    flags = OPERAND_FLAGS[operands] if code == VAE_DTYPE_BF16 else 0
    if norm_in_conv:
        flags |= VAE_DECODE_NORM_IN_CONV
    dec = Decoder(code, lc, spec["groups"], spec["eps"], layers, flat, act_dtype=act,
                  flags=flags)
    if packed:
        dec.pack_weights(device)
    return dec
