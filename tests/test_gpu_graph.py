"""The decode captured in a HIP graph and replayed.

vae_decode_tiled enqueues kernels only: no allocation, copy, memset, event or synchronisation
(with op timing off). A caller can therefore capture a whole decode, every layer of every
patch or tile, in one graph and replay it with a single launch. Each replay below runs after
eager work that overwrites the output and the whole workspace, and must equal the eager decode
bit for bit.
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


@pytest.mark.parametrize("mode", ["patch", "overlap"])
def test_decode_replays_from_a_hip_graph(v, mode):
    import torch
    spec = vae_synth.LTX2_TINY
    z = ndhwc(vae_synth.latent(spec))
    zd = dev(z, spec["dtype"])
    dec = v.upload_decoder(spec, vae_synth.decoder_params(spec))
    if mode == "patch":
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=(1, 2))
    else:
        desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, z.shape, spec["scale"],
                             tile=spec["overlap_tile"], stride=spec["overlap_stride"])
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
