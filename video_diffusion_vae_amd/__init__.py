"""Tiled, halo-extended decode of a causal 3-D video VAE on AMD MI355X (gfx950).

The compute lives in libvae_mi355x.so (HIP kernels behind the C ABI in include/vae.h). This package
is its ctypes binding plus parameter upload helpers; importing it fails when the library is not
built.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (LIB, EXPORTS, Decoder, VaeError, tensor_desc, tiling_desc,  # noqa: F401
                       last_error_info, layer_descs)
from .weights import upload_decoder, conv_weight_layout, latent_channels, pad_latent  # noqa: F401
