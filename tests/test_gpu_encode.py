"""GPU parity of the encode path against the CPU oracle, through the C ABI.

- vae_space_to_depth: a permutation, so bit-exact against oracle.space_to_depth for every dtype
  and vector width (16-byte, 8-byte and scalar rows);
- the LTX-2-shaped encoder plan, untiled (vae_decode_tiled with a 1 x 1 patch grid), against
  oracle.encode, and in overlap tiles cut on the latent grid (down = the plan's folds) against
  oracle.encode_overlap_blend, at the bf16 bar: PSNR >= 50 dB and max-abs <= 2e-2 on the latent. The 3-channel video is padded with a zero channel on upload (4 x 16 = 64 channels after
  the patchify fold) and conv_in gets zero weights there, so the sums are the same.
"""
import functools

import numpy as np
import pytest

import oracle
import vae_synth
from _util import ndhwc, dev, host, psnr, round_f16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def v():
    import torch
    import video_diffusion_vae_amd as v
    assert torch.cuda.is_available()
    return v


S2D_CASES = [
    # (N, T, H, W, C), dtype, (st, sh, sw)
    ((1, 9, 16, 24, 4), "bf16", (1, 4, 4)),      # the patchify of a padded video: pairs of
                                                 # sub-positions in 16-byte vectors
    ((1, 5, 8, 12, 2), "f32", (2, 2, 2)),        # fp32 pairs, causal front copy
    ((2, 4, 6, 8, 4), "f16", (1, 2, 4)),         # fp16 pairs, two samples
    ((1, 3, 4, 6, 4), "bf16", (2, 2, 1)),        # sw odd: 8-byte vectors
    ((1, 5, 8, 12, 32), "f32", (2, 2, 2)),       # 16-byte vectors, causal front copy
    ((2, 3, 4, 6, 64), "bf16", (2, 2, 2)),
    ((1, 9, 6, 10, 3), "f32", (4, 2, 1)),        # scalar rows, three front copies
    ((1, 4, 6, 6, 8), "f16", (1, 3, 2)),
    ((1, 1, 2, 2, 16), "bf16", (1, 1, 1)),       # identity fold
]


@pytest.mark.parametrize("case", S2D_CASES)
def test_space_to_depth_bit_exact(v, case):
    import torch
    shape, dt, fold = case
    st, sh, sw = fold
    x = vae_synth.normal(shape, [60, shape[-1]], dtype=dt)
    if dt == "f16":
        x = round_f16(x)
    ref = oracle.space_to_depth(x, st, sh, sw)
    xd = dev(x, dt)
    y = torch.full(ref.shape, -7.0, device="cuda", dtype=xd.dtype)
    v.vae_space_to_depth(xd, st, sh, sw, y)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), ref)


def test_space_to_depth_argument_rules(v):
    import torch
    x = torch.zeros((1, 4, 8, 8, 4), device="cuda", dtype=torch.bfloat16)
    y = torch.zeros((1, 2, 4, 4, 32), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(v.VaeError) as e:         # 4 frames do not fold causally by 2
        v.vae_space_to_depth(x, 2, 2, 2, y)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 1
    with pytest.raises(v.VaeError) as e:         # y of the wrong shape (16 channels, not 32)
        v.vae_space_to_depth(x[:, :3], 2, 2, 2, y[..., :16].contiguous())
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    v.vae_space_to_depth(x[:, :3], 2, 2, 2, y)   # 3 frames fold to 2: accepted
    with pytest.raises(v.VaeError) as e:         # dtype mismatch
        v.vae_space_to_depth(x[:, :3], 2, 2, 2, y.float())
    assert e.value.status == v.VAE_ERR_INVALID_ARG


@functools.lru_cache(maxsize=None)
def _params(name):
    return vae_synth.decoder_params(vae_synth.WORKLOADS[name], affine_seed=9)


@functools.lru_cache(maxsize=None)
def _oracle(name, tiles=None):
    spec = vae_synth.WORKLOADS[name]
    x = ndhwc(vae_synth.latent(spec))
    if tiles is None:
        return oracle.encode(spec, x, _params(name))
    return oracle.encode_overlap_blend(spec, x, _params(name), tiles[0], tiles[1])


def _encode(v, name, operands="f16", repeat=1, tiles=None, patches=None, launch="merged"):
    import torch
    spec = vae_synth.WORKLOADS[name]
    x = ndhwc(vae_synth.latent(spec))
    xp = v.pad_latent(x, spec)
    enc = v.upload_decoder(spec, _params(name), operands=operands)
    enc.set_launch(v.VAE_LAUNCH_PER_PATCH if launch == "per_patch" else v.VAE_LAUNCH_MERGED)
    xd = dev(xp, "bf16")
    if patches is not None:
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, xp.shape, (1, 1, 1), patches=patches,
                             down=spec["down"])
    elif tiles is None:
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, xp.shape, (1, 1, 1))
    else:
        desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, xp.shape, (1, 1, 1), tile=tiles[0],
                             stride=tiles[1], down=spec["down"])
    ws = torch.empty(enc.workspace_size(desc), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(repeat):
        out = torch.full(oracle.output_shape(spec, x.shape), float("nan"), device="cuda",
                         dtype=torch.float32)
        enc.vae_decode_tiled(xd, desc, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    enc.close()
    return outs if repeat > 1 else outs[0]


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("name", ["ltx2_enc_tiny", "ltx2_enc_small"])
def test_encode_untiled_matches_oracle(v, name, operands):
    got = host(_encode(v, name, operands))
    ref = _oracle(name)
    assert got.shape == ref.shape
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


@pytest.mark.parametrize("name,tiles", [("ltx2_enc_small", ((2, 3), (2, 2))),
                                        ("ltx2_enc_tiny", ((2, 2), (1, 1))),
                                        ("ltx2_enc_tiny", ((1, 2), (1, 1)))])
def test_encode_overlap_blend_matches_oracle(v, name, tiles):
    """Tiles cut on the latent grid, each encoding its pixel crop alone (own borders, own
    GroupNorm statistics), blended in latent space: against oracle.encode_overlap_blend."""
    got = host(_encode(v, name, tiles=tiles))
    ref = _oracle(name, tiles)
    assert got.shape == ref.shape
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


@pytest.mark.parametrize("name,patches", [("ltx2_enc_small", (2, 2)), ("ltx2_enc_tiny", (1, 3))])
def test_encode_patch_halo_matches_untiled_oracle(v, name, patches):
    """Bands in whole multiples of the 32-pixel fold; halos read in place and GroupNorm statistics
    merged across patches: the untiled encode."""
    got = host(_encode(v, name, patches=patches))
    ref = _oracle(name)
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


def test_encode_one_overlap_tile_is_the_untiled_encode(v):
    import torch
    whole = _encode(v, "ltx2_enc_small")
    one = _encode(v, "ltx2_enc_small", tiles=((8, 8), (8, 8)))
    assert torch.equal(whole, one)


def test_encode_is_deterministic(v):
    import torch
    a, b = _encode(v, "ltx2_enc_tiny", repeat=2)
    assert torch.equal(a, b)


@pytest.mark.parametrize("tile,stride", [((2, 3), (1, 2)), ((3, 2), (2, 2))])
def test_tile_merge_with_an_encoder_desc(v, tile, stride):
    """vae_tile_merge under an encoder desc (down = 8, 32, 32): the tiles are latent boxes, the
    weight sums come from the latent grid, so blending exact crops of a latent gives it back."""
    import torch
    t, h, w = 17, 4 * 32, 5 * 32                      # latent [3, 4, 5]
    desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, t, h, w, 4), (1, 1, 1), tile=tile,
                         stride=stride, down=(8, 32, 32))
    tiles = v.vae_tile_split(desc)
    lat = vae_synth.normal((1, 3, 4, 5, 6), [61]).astype(np.float64)
    out = torch.full(lat.shape, 3.0, device="cuda", dtype=torch.float32)
    for k, tl in enumerate(tiles):
        o = tl.out
        crop = lat[:, o.t0:o.t1, o.h0:o.h1, o.w0:o.w1]
        flags = (v.VAE_MERGE_ZERO if k == 0 else 0) | \
                (v.VAE_MERGE_FINALIZE if k == len(tiles) - 1 else 0)
        v.vae_tile_merge(dev(crop, "f32"), tl, desc, out, flags)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(out), lat, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("patches", [None, (1, 4)])
def test_ltx2_720p_encode_against_golden(v, patches):
    """The full LTX-2-shaped 720p encode ([1,3,121,704,1280] -> [1,16,22,40,256]), untiled and in
    1 x 4 patch-halo bands, at the latent positions the oracle's fp64 encode stored
    (tests/golden/make_ltx2_enc_720p_samples.py), all 256 channels each."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "ltx2_enc_720p_samples.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    g = np.load(path)
    spec = vae_synth.LTX2_ENC_720P
    import torch
    x = ndhwc(vae_synth.latent(spec))
    xp = v.pad_latent(x, spec)
    enc = v.upload_decoder(spec, vae_synth.decoder_params(spec, affine_seed=9))
    xd = dev(xp, "bf16")
    del x, xp
    if patches is None:
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, xd.shape, (1, 1, 1))
    else:
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, xd.shape, (1, 1, 1), patches=patches,
                             down=spec["down"])
    ws = torch.empty(enc.workspace_size(desc), dtype=torch.uint8, device="cuda")
    out = torch.full(tuple(int(d) for d in g["shape"]), float("nan"), device="cuda",
                     dtype=torch.float32)
    enc.vae_decode_tiled(xd, desc, out, ws)
    torch.cuda.synchronize()
    enc.close()
    del ws, xd
    pos = g["positions"]
    got = out[0, pos[:, 0], pos[:, 1], pos[:, 2], :].double().cpu().numpy()
    ref = g["values"].astype(np.float64)
    assert np.all(np.isfinite(got))
    p = 10 * np.log10((float(g["out_max"]) - float(g["out_min"])) ** 2 / np.mean((got - ref) ** 2))
    m = float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)
    o = out.double()
    assert abs(float(o.mean()) - float(g["out_mean"])) <= 1e-3 * float(g["out_std"])
    assert abs(float(o.std()) / float(g["out_std"]) - 1.0) <= 1e-3


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("name,mode", [("ltx2_enc_strided_tiny", "untiled"),
                                       ("ltx2_enc_strided_tiny", "patch"),
                                       ("ltx2_enc_strided_tiny", "per_patch"),
                                       ("ltx2_enc_strided_tiny", "overlap"),
                                       ("wan_enc_tiny", "untiled"),
                                       ("wan_enc_tiny", "patch"),
                                       ("wan_enc_tiny", "per_patch"),
                                       ("wan_enc_tiny", "overlap")])
def test_strided_encoders_match_oracle(v, name, mode, operands):
    """Encoders whose downsamplers are strided causal convs (stride 2 with zero padding around,
    LTX-2's bare kind; padding after the image, the Wan kind), untiled, in patch bands of whole
    folds (one launch per layer, or one per patch), and in latent-grid overlap tiles, against the
    oracle at the bf16 bar."""
    spec = vae_synth.WORKLOADS[name]
    if mode == "overlap":
        tiles = (spec["overlap_tile"], spec["overlap_stride"])
        got = host(_encode(v, name, operands, tiles=tiles))
        ref = _oracle(name, tiles)
    else:
        patches = None if mode == "untiled" else spec["patch_grid"]
        got = host(_encode(v, name, operands, patches=patches,
                           launch="per_patch" if mode == "per_patch" else "merged"))
        ref = _oracle(name)
    assert got.shape == ref.shape
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)
