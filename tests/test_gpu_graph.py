"""The decode (and the encode) captured in a HIP graph and replayed.

vae_decode_tiled enqueues kernels only: no allocation, copy, memset, event or synchronisation
(with op timing off). A caller can therefore capture a whole decode, every layer of every
patch, tile or causal clip, in one graph and replay it with a single launch. Each replay below
runs after eager work that overwrites the output and the whole workspace, and must equal the
eager decode bit for bit.
"""
import pytest

import oracle
import vae_synth
from _util import ndhwc, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def v():
    import torch
    import video_diffusion_vae_amd as v
    assert torch.cuda.is_available()
    return v


CASES = [
    # (plan, tiling, tiling arguments)
    ("ltx2_tiny", "patch", dict(patches=(1, 2))),
    ("ltx2_tiny", "overlap", {}),
    ("ltx2_mid", "overlap", dict(tile_t=2, stride_t=1)),           # temporal tiles as well
    ("ltx2_enc_small", "patch", dict(patches=(1, 1))),             # the encoder, untiled
    ("ltx2_enc_small", "patch", dict(patches=(2, 2), down=(8, 32, 32))),
    ("ltx2_enc_small", "overlap", dict(down=(8, 32, 32))),         # latent-grid tiles
    # every conv, GroupNorm pass and upsampling launched per patch box
    ("ltx2_tiny", "patch", dict(patches=(2, 2), launch="per_patch")),
    # causal clips, each conv carrying its last two input frames (merged and per patch)
    ("wan_tiny", "patch", dict(patches=(2, 2), clip=1)),
    ("wan_tiny", "patch", dict(patches=(2, 2), clip=2, launch="per_patch")),
]


@pytest.mark.parametrize("name,mode,kw", CASES)
def test_decode_replays_from_a_hip_graph(v, name, mode, kw):
    import torch
    spec = vae_synth.WORKLOADS[name]
    z = ndhwc(vae_synth.latent(spec))
    zp = v.pad_latent(z, spec)
    zd = dev(zp, spec["dtype"])
    dec = v.upload_decoder(spec, vae_synth.decoder_params(spec))
    kw = dict(kw)
    if kw.pop("launch", None) == "per_patch":
        dec.set_launch(v.VAE_LAUNCH_PER_PATCH)
    if "clip" in kw:
        dec.set_clip_frames(kw.pop("clip"))
    scale = spec.get("scale", (1, 1, 1))
    if mode == "patch":
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, zp.shape, scale, **kw)
    else:
        desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, zp.shape, scale,
                             tile=spec["overlap_tile"], stride=spec["overlap_stride"], **kw)
    ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
    shape = oracle.output_shape(spec, z.shape)
    eager = torch.empty(shape, dtype=torch.float32, device="cuda")
    dec.vae_decode_tiled(zd, desc, eager, ws)
    torch.cuda.synchronize()

    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the default stream, as capture needs
        dec.vae_decode_tiled(zd, desc, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dec.vae_decode_tiled(zd, desc, out, ws)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xA5 + k)                  # stale workspace contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {k}"
    del graph
    dec.close()
