"""CPU oracle for the tiled, halo-extended decode of a causal 3-D video VAE.

TEST INFRASTRUCTURE. This package is the plain, slow and obviously correct statement of what the
decode computes. Only these may import, call or run anything in it:
- the tests;
- the smoke check in ``__graft_entry__``;
- the CPU-baseline leg of ``bench.py``.
The GPU library never does, and it shares no code, headers, tables or helpers with this package.
The only thing both sides read is the seeded input module ``vae_synth``.

Conventions:
- every array is channels-last, ``[N, T, H, W, C]``;
- all arithmetic is float64;
- inputs arrive as float32 (bf16-exact for bf16 workloads) and are upcast exactly.

Sources, cited by page title and the part of the page:
- "[TRTLLM-14029][feat] LTX-2 tile-parallel VAE decode" (TensorRT-LLM PR #15753): serial and
  tile-parallel tiled decode, the blend mask built from per-axis parts, the weight buffer and the
  final divide (Description and Approach).
- "[Feature] Support VAE tiling parallel encode for LTX-2" (vllm-omni PR #4831): tile grid rule
  (tile 512, stride 448, ratio 32; 576 -> 512 + 128) and split -> exec -> merge (Purpose; review
  thread).
- "Add tiled VAE parallelism & extended model support" (DistVAE PR #14): patch sharding with halo
  rows, global-mean biased-variance GroupNorm across patches, band rule, padding at true borders
  only, causal temporal padding by repeated frames, depth-to-space upsampler, RMS norms that reduce
  over channels and a mid-block attention that takes each frame whole (commit messages).

Parity status of each function:
- pinned by tests/test_oracle_*.py: conv (brute force, torch CPU, causality), GroupNorm (torch CPU,
  closed forms, Chan split invariance, negative control), SiLU identities, upsampling (repeat,
  inverse), tiling (page-printed grids, band rule), merge identities, mode A == whole decode,
  mode B 1x1 == whole decode; RMS norm (closed forms, torch CPU rms_norm), frame attention (torch
  CPU scaled_dot_product_attention, uniform-attention and permutation invariants); the encode
  path (space_to_depth by brute force and its inverse, patch-halo encode == whole, fold-only
  tiled encodes == whole, the strided causal conv against torch CPU conv3d and brute force);
- parity unpinned: the absolute output values of a full random-init decoder. The pages print no
  tensor values, so a decoder's output is pinned only through its parts and the invariants above.
"""
from .layers import (causal_conv3d, strided_causal_conv3d, conv3d_valid, causal_time_pad,
                     group_norm, silu,
                     nearest_upsample, depth_to_space, space_to_depth, rms_norm, softmax,
                     frame_attention)
from .stats import group_moments, chan_combine, normalize_with
from .tiling import (bands, axis_tiles, patch_tiles, overlap_tiles, ramp_1d, axis_weight_sum)
from .decoder import (decode, decode_patch_halo, decode_overlap_blend, merge_tiles,
                      output_shape, encode, encode_patch_halo, encode_overlap_blend,
                      decode_causal_clips)

__all__ = [
    "causal_conv3d", "strided_causal_conv3d", "conv3d_valid", "causal_time_pad", "group_norm",
    "silu", "nearest_upsample",
    "depth_to_space", "space_to_depth", "rms_norm", "softmax", "frame_attention",
    "group_moments", "chan_combine", "encode", "encode_patch_halo", "encode_overlap_blend",
    "normalize_with", "bands", "axis_tiles",
    "patch_tiles", "overlap_tiles", "ramp_1d", "axis_weight_sum", "decode", "decode_patch_halo",
    "decode_overlap_blend", "merge_tiles", "output_shape", "decode_causal_clips",
]
