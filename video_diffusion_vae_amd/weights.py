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
    flat = []
    for p in params:
        if p["kind"] == "conv":
            flat.append(conv_weight_layout(p["w"], tdt, device))
            flat.append(torch.as_tensor(np.asarray(p["b"], np.float32)).to(device))
        else:
            flat.append(torch.as_tensor(np.asarray(p["gamma"], np.float32)).to(device))
            flat.append(torch.as_tensor(np.asarray(p["beta"], np.float32)).to(device))
    code = VAE_DTYPE_BF16 if spec["dtype"] == "bf16" else VAE_DTYPE_F32
    act = VAE_DTYPE_BF16 if act_dtype == "bf16" else VAE_DTYPE_F32
    flags = OPERAND_FLAGS[operands] if code == VAE_DTYPE_BF16 else 0
    dec = Decoder(code, spec["latent"][1], spec["groups"], spec["eps"], spec["layers"], flat,
                  act_dtype=act, flags=flags)
    if packed:
        dec.pack_weights(device)
    return dec
