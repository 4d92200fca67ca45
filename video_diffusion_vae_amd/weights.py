"""Upload a decoder's parameters to the device in the library's layouts.

This is setup-time marshalling, not part of the decode itself:
- conv weights go from [Cout, Cin, 3, 3, 3] to [Cout, 3, 3, 3, Cin] (the K dimension, taps then
  channels, contiguous per output channel);
- biases, gamma and beta become fp32 vectors.
"""
from __future__ import annotations

import numpy as np

from ._binding import (Decoder, VAE_DTYPE_BF16, VAE_DTYPE_F32, VAE_DECODE_F16_OPERANDS,
                       VAE_DECODE_SPLIT_FP32_OPERANDS)

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


def latent_channels(spec: dict) -> int:
    """Channels of the latent the GPU decoder takes: the plan's, rounded up to a multiple of 32
    for a bf16 plan, so that the first conv runs on the matrix cores (48 -> 64 for the Wan-shaped
    plan). The extra channels are zeros in the latent and in the first conv's weights, so the
    result is the same sum."""
    c = spec["latent"][1]
    return (c + 31) // 32 * 32 if spec["dtype"] == "bf16" else c


def pad_latent(z, spec: dict):
    """NDHWC host latent padded with zero channels to latent_channels(spec)."""
    c = latent_channels(spec)
    if z.shape[-1] == c:
        return z
    pad = np.zeros(z.shape[:-1] + (c - z.shape[-1],), dtype=z.dtype)
    return np.concatenate([z, pad], axis=-1)


def upload_decoder(spec: dict, params: list, device="cuda", act_dtype="f32", operands="f16",
                   packed=True):
    """Build a Decoder for a layer plan ``spec`` with parameter dicts in plan order.

    Each parameter dict is {"kind": "conv", "w", "b"} or {"kind": "gn", "gamma", "beta"} holding
    host arrays. ``act_dtype`` is the storage dtype of the activations between ops ("f32" or
    "bf16"). ``operands`` picks how convs that read an fp32 activation get their operands
    (OPERAND_FLAGS; bf16 plans only). ``packed`` gives the MFMA convs fragment-packed weight
    copies. Returns the Decoder; it keeps the device tensors alive.
    """
    import torch
    tdt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
    f32 = lambda a: torch.as_tensor(np.asarray(a, np.float32)).to(device)
    lc = latent_channels(spec)
    layers = [dict(op) for op in spec["layers"]]
    flat = []
    for k, p in enumerate(params):
        if p["kind"] == "conv":
            w = np.asarray(p["w"], np.float32)
            if k == 0 and w.shape[1] < lc:       # zero weights for the zero latent channels
                w = np.concatenate([w, np.zeros((w.shape[0], lc - w.shape[1]) + w.shape[2:],
                                                np.float32)], axis=1)
                layers[0]["cin"] = lc
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
    dec = Decoder(code, lc, spec["groups"], spec["eps"], layers, flat, act_dtype=act,
                  flags=flags)
    if packed:
        dec.pack_weights(device)
    return dec
