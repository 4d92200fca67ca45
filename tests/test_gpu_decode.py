"""GPU parity of the whole decode (vae_decode_tiled) against the CPU oracle.

Tolerances:
- fp32 workloads (the single conv+GN workload, the tiny decoder): relative max-abs <= 1e-4;
- bf16 workloads: PSNR >= 50 dB and max-abs <= 2e-2 against the fp64 oracle on the same
  bf16-exact inputs and weights.
Patch-halo decodes are compared with the oracle's untiled decode, which they must equal.
Overlap-blend decodes are compared with the oracle's overlap-blend decode.
"""
import functools
import os

import numpy as np
import pytest

import oracle
import vae_synth
from _util import ndhwc, dev, host, rel_max_abs, psnr

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def v():
    import torch
    import video_diffusion_vae_amd as v
    assert torch.cuda.is_available()
    return v


CONV_GN_PLAN = {
    "name": "conv_gn_32", "dtype": "f32", "latent": vae_synth.CONV_GN["input"], "groups": 8,
    "eps": 1e-6, "layers": [{"op": "conv", "cin": 32, "cout": 32}, {"op": "gn_silu"}],
    "scale": (1, 1, 1),
}


def params_of(name, affine=None):
    # the LTX-2-shaped workloads share one layer plan, hence one weight set (as do the tiny ones)
    if name.startswith("ltx2_tiny"):
        key = "ltx2_tiny"
    elif name.startswith("ltx2_"):
        key = "ltx2_720p"
    else:
        key = name
    return _params(key, affine)


@functools.lru_cache(maxsize=None)
def _params(name, affine):
    spec = CONV_GN_PLAN if name == "conv_gn_32" else vae_synth.WORKLOADS[name]
    return vae_synth.decoder_params(spec, affine_seed=affine)


def spec_of(name):
    return CONV_GN_PLAN if name == "conv_gn_32" else vae_synth.WORKLOADS[name]


@functools.lru_cache(maxsize=None)
def oracle_out(name, mode, affine=None, tt=(0, 0)):
    spec = spec_of(name)
    z = ndhwc(vae_synth.latent(spec))
    p = params_of(name, affine)
    if mode == "whole":
        return oracle.decode(spec, z, p)
    return oracle.decode_overlap_blend(spec, z, p, spec["overlap_tile"], spec["overlap_stride"],
                                       spec["scale"], tt[0], tt[1])


def gpu_decode(v, name, mode, patches=(1, 1), affine=None, repeat=1, act="f32", operands="f16",
               tt=(0, 0), launch="merged", timing=None):
    """Decode through vae_decode_tiled. ``operands``: how convs reading an fp32 activation get
    their operands, "f16" (the default), "split" (bf16 hi + lo) or "bf16". ``tt``: temporal tile
    and stride of an overlap-blend decode (0: T whole). ``launch``: "merged" (one launch per
    layer) or "per_patch" (every conv, GroupNorm pass and upsampling once per patch box).
    ``timing``: a list that receives the per-op records of the last decode."""
    import torch
    spec = spec_of(name)
    z = ndhwc(vae_synth.latent(spec))
    dec = v.upload_decoder(spec, params_of(name, affine), act_dtype=act, operands=operands)
    dec.set_launch(v.VAE_LAUNCH_PER_PATCH if launch == "per_patch" else v.VAE_LAUNCH_MERGED)
    if timing is not None:
        dec.set_timing(True)
    zd = dev(z, spec["dtype"])
    if mode == "patch":
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=patches)
    else:
        desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, z.shape, spec["scale"],
                             tile=spec["overlap_tile"], stride=spec["overlap_stride"],
                             tile_t=tt[0], stride_t=tt[1])
    ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
    out_shape = oracle.output_shape(spec, z.shape)
    outs = []
    for _ in range(repeat):
        out = torch.full(out_shape, float("nan"), device="cuda", dtype=torch.float32)
        dec.vae_decode_tiled(zd, desc, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    if timing is not None:
        timing.extend(dec.timing())
    dec.close()
    return outs if repeat > 1 else outs[0]


@pytest.mark.parametrize("patches", [(1, 1), (1, 2), (2, 1)])
@pytest.mark.parametrize("affine", [None, 4])
def test_conv_gn_workload(v, patches, affine):
    """One causal conv 32->32 + GN(8) + SiLU on [1,32,5,32,32], whole and as width patches."""
    got = host(gpu_decode(v, "conv_gn_32", "patch", patches, affine))
    assert rel_max_abs(got, oracle_out("conv_gn_32", "whole", affine)) <= 1e-4


@pytest.mark.parametrize("patches", [(1, 1), (2, 2), (1, 3)])
def test_tiny_decoder_patch_halo(v, patches):
    got = host(gpu_decode(v, "tiny_decoder", "patch", patches, affine=3))
    assert got.shape == (1, 5, 64, 64, 3)
    assert rel_max_abs(got, oracle_out("tiny_decoder", "whole", 3)) <= 1e-4


def test_tiny_decoder_overlap_blend(v):
    got = host(gpu_decode(v, "tiny_decoder", "overlap", affine=3))
    assert rel_max_abs(got, oracle_out("tiny_decoder", "overlap", 3)) <= 1e-4


@pytest.mark.parametrize("tt", [(2, 1), (3, 2)])
def test_tiny_decoder_overlap_blend_temporal_tiles(v, tt):
    """Tiles in T as well: (2, 1) cuts the 3 latent frames into clips [0,2) [1,3) [2,3), the last
    a single frame; (3, 2) leaves T whole (no longer than the tile)."""
    got = host(gpu_decode(v, "tiny_decoder", "overlap", affine=3, tt=tt))
    ref = oracle_out("tiny_decoder", "overlap", 3, tt)
    assert got.shape == ref.shape == (1, 5, 64, 64, 3)
    assert rel_max_abs(got, ref) <= 1e-4
    if tt == (3, 2):
        assert rel_max_abs(got, oracle_out("tiny_decoder", "overlap", 3)) <= 1e-4


def _bf16_bar(got, ref):
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)
    return p, m


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("name,patches", [("ltx2_small", (1, 2)), ("ltx2_small", (1, 1)),
                                          ("ltx2_mid", (2, 3))])
def test_ltx2_shaped_patch_halo(v, name, patches, operands):
    got = host(gpu_decode(v, name, "patch", patches, operands=operands))
    _bf16_bar(got, oracle_out(name, "whole"))


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("name", ["ltx2_small", "ltx2_mid"])
def test_ltx2_shaped_overlap_blend(v, name, operands):
    got = host(gpu_decode(v, name, "overlap", operands=operands))
    _bf16_bar(got, oracle_out(name, "overlap"))


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("mode,patches", [("patch", (1, 4)), ("overlap", (1, 1))])
def test_ltx2_720p_one_frame_every_value(v, mode, patches, operands):
    """The full-width 720p plan on one latent frame ([1,128,1,22,40] -> [1,1,704,1280,3]): every
    one of the 2.7M output values against the oracle, in both tiling modes and with fp16 or split
    operands for the convs that read an fp32 activation."""
    got = host(gpu_decode(v, "ltx2_720p_1f", mode, patches, operands=operands))
    assert got.shape == (1, 1, 704, 1280, 3)
    _bf16_bar(got, oracle_out("ltx2_720p_1f", "whole" if mode == "patch" else "overlap"))


def test_no_split_on_every_conv_matches_unsplit_decoder(v):
    """Per-conv no_split set on every conv of a splitting decoder gives, bit for bit, the decoder
    without the split flag."""
    import copy
    import torch
    spec = vae_synth.LTX2_TINY
    ns = copy.deepcopy(spec)
    for op in ns["layers"]:
        if op["op"] == "conv":
            op["no_split"] = True
    z = ndhwc(vae_synth.latent(spec))
    zd = dev(z, "bf16")
    desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=(1, 2))
    outs = []
    for sp, operands in ((ns, "split"), (spec, "bf16")):
        dec = v.upload_decoder(sp, params_of("ltx2_tiny"), operands=operands)
        ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
        out = torch.empty(oracle.output_shape(spec, z.shape), dtype=torch.float32, device="cuda")
        dec.vae_decode_tiled(zd, desc, out, ws)
        torch.cuda.synchronize()
        outs.append(out)
        dec.close()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("name", ["ltx2_small", "ltx2_tiny"])
def test_decode_is_deterministic(v, name, operands):
    """Two decodes through one workspace are bit-identical (ltx2_tiny's last stage is 32 channels
    wide, so half of each 64-wide conv tile lies past Cout)."""
    import torch
    a, b = gpu_decode(v, name, "patch", (1, 2), repeat=2, operands=operands)
    assert torch.equal(a, b)
    a, b = gpu_decode(v, name, "overlap", repeat=2, operands=operands)
    assert torch.equal(a, b)


def _golden(mode):
    path = os.path.join(GOLDEN, f"ltx2_720p_{mode}_samples.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    return np.load(path)


def _check_golden(g, out):
    pos = g["positions"]
    got = out[0, pos[:, 0], pos[:, 1], pos[:, 2], :].double().cpu().numpy()
    ref = g["values"]
    assert np.all(np.isfinite(got))
    p = 10 * np.log10((float(g["out_max"]) - float(g["out_min"])) ** 2 /
                      np.mean((got - ref) ** 2))
    m = float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)
    o = out.double()
    assert abs(float(o.mean()) - float(g["out_mean"])) <= 1e-3 * float(g["out_std"])
    assert abs(float(o.std()) / float(g["out_std"]) - 1.0) <= 1e-3


@pytest.mark.parametrize("operands", ["f16", "split"])
def test_ltx2_720p_overlap_blend_against_golden(v, operands):
    """Full 720p overlap-blend decode: 2x3 tiles of 16x16 latents, stride 14 (512/448 px)."""
    g = _golden("overlap")
    _check_golden(g, gpu_decode(v, "ltx2_720p", "overlap", operands=operands))


@pytest.mark.parametrize("operands", ["f16", "split"])
def test_ltx2_720p_patch_halo_against_golden(v, operands):
    """Full 720p decode (latent [1,128,16,22,40] -> [1,121,704,1280,3]), 1x4 width patches, at
    the pixels the oracle's full fp64 decode stored."""
    g = _golden("whole")
    out = gpu_decode(v, "ltx2_720p", "patch", (1, 4), operands=operands)
    pos = g["positions"]
    got = out[0, pos[:, 0], pos[:, 1], pos[:, 2], :].double().cpu().numpy()
    ref = g["values"]
    assert np.all(np.isfinite(got))
    p = 10 * np.log10((float(g["out_max"]) - float(g["out_min"])) ** 2 /
                      np.mean((got - ref) ** 2))
    m = float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)
    o = out.double()
    assert abs(float(o.mean()) - float(g["out_mean"])) <= 1e-3 * float(g["out_std"])
    assert abs(float(o.std()) / float(g["out_std"]) - 1.0) <= 1e-3


@pytest.mark.parametrize("launch", ["merged", "per_patch"])
def test_ltx2_720p_full_decode_band_every_value(v, launch):
    """The full 720p decode (16 latent frames, GroupNorm statistics over all 121 output frames),
    1x4 width patches: every value of a 16-row band of output frame 60, all 1280 columns (the
    three patch seams inside it), against the oracle's full fp64 decode
    (tests/golden/make_ltx2_720p_samples.py band)."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "ltx2_720p_whole_band.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    g = np.load(path)
    f, (r0, r1) = int(g["frame"]), (int(x) for x in g["rows"])
    out = gpu_decode(v, "ltx2_720p", "patch", (1, 4), launch=launch)
    assert tuple(out.shape) == tuple(int(d) for d in g["shape"])
    got = out[0, f, r0:r1].double().cpu().numpy()
    ref = g["values"]
    assert got.shape == ref.shape == (16, 1280, 3)
    p = 10 * np.log10((float(g["out_max"]) - float(g["out_min"])) ** 2 /
                      np.mean((got - ref) ** 2))
    m = float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


def test_ltx2_tiny_both_modes(v):
    got = host(gpu_decode(v, "ltx2_tiny", "patch", (1, 2)))
    _bf16_bar(got, oracle_out("ltx2_tiny", "whole"))
    got = host(gpu_decode(v, "ltx2_tiny", "overlap"))
    _bf16_bar(got, oracle_out("ltx2_tiny", "overlap"))


@pytest.mark.parametrize("mode,patches", [("patch", (1, 2)), ("overlap", (1, 1))])
def test_ltx2_tiny_batch_of_two(v, mode, patches):
    """N = 2: statistics, tiles and epilogue offsets per sample."""
    got = host(gpu_decode(v, "ltx2_tiny_n2", mode, patches))
    assert got.shape[0] == 2
    _bf16_bar(got, oracle_out("ltx2_tiny_n2", "whole" if mode == "patch" else "overlap"))


@pytest.mark.parametrize("operands", ["f16", "split"])
def test_packed_and_standard_weights_decode_identically(v, operands):
    import torch
    spec = vae_synth.LTX2_TINY
    z = ndhwc(vae_synth.latent(spec))
    zd = dev(z, "bf16")
    desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=(1, 2))
    outs = []
    for packed in (False, True):
        dec = v.upload_decoder(spec, params_of("ltx2_tiny"), packed=packed, operands=operands)
        ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
        out = torch.empty(oracle.output_shape(spec, z.shape), dtype=torch.float32, device="cuda")
        dec.vae_decode_tiled(zd, desc, out, ws)
        torch.cuda.synchronize()
        outs.append(out)
        dec.close()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("name,patches,launch,operands", [
    ("ltx2_tiny", (1, 2), "merged", "f16"),
    ("ltx2_tiny", (2, 2), "per_patch", "f16"),
    ("ltx2_tiny", (1, 2), "merged", "bf16"),
    ("ltx2_tiny_n2", (1, 1), "merged", "f16"),
    ("mixed_rms_gn", (1, 2), "per_patch", "f16"),
    ("mixed_rms_gn", (1, 1), "merged", "bf16"),
])
def test_norm_in_conv_staging_decodes_identically(v, name, patches, launch, operands):
    """With VAE_DECODE_NORM_IN_CONV every GroupNorm that a packed MFMA conv can apply while
    staging (both norms of each residual block, the GN_SILU before conv_out) gives the decode of
    separate normalise passes bit for bit, with no normalise pass left."""
    import torch
    spec = spec_of(name)
    z = ndhwc(vae_synth.latent(spec))
    zd = dev(z, "bf16")
    desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=patches)
    outs, kinds = [], []
    for fused in (False, True):
        dec = v.upload_decoder(spec, params_of(name), operands=operands, norm_in_conv=fused)
        if launch == "per_patch":
            dec.set_launch(v.VAE_LAUNCH_PER_PATCH)
        dec.set_timing(True)
        ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
        out = torch.full(oracle.output_shape(spec, z.shape), float("nan"), dtype=torch.float32,
                         device="cuda")
        dec.vae_decode_tiled(zd, desc, out, ws)
        torch.cuda.synchronize()
        gn_bytes = sum(r["bytes"] for r in dec.timing() if r["kind"] == "gn")
        outs.append(out)
        kinds.append(gn_bytes)
        dec.close()
    assert torch.equal(outs[0], outs[1])
    assert kinds[1] < kinds[0]        # the normalise passes are gone
    _bf16_bar(host(outs[1]), oracle_out(name, "whole"))


# ------------------------------------------------------------------------------------------------
# Per-patch launches: every conv, GroupNorm pass and upsampling once per patch box, over that box
# only, with the GroupNorm statistics merged across the boxes (one rank's share of a patch split).
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("patches", [(1, 2), (2, 1), (2, 2)])
def test_conv_gn_workload_per_patch(v, patches):
    got = host(gpu_decode(v, "conv_gn_32", "patch", patches, 4, launch="per_patch"))
    assert rel_max_abs(got, oracle_out("conv_gn_32", "whole", 4)) <= 1e-4


@pytest.mark.parametrize("patches", [(2, 2), (1, 3), (3, 1)])
def test_tiny_decoder_per_patch(v, patches):
    """fp32: the per-patch decode equals the oracle's whole decode (rel 1e-4) and the merged
    launches up to the rounding order of the statistics."""
    got = host(gpu_decode(v, "tiny_decoder", "patch", patches, affine=3, launch="per_patch"))
    assert rel_max_abs(got, oracle_out("tiny_decoder", "whole", 3)) <= 1e-4
    merged = host(gpu_decode(v, "tiny_decoder", "patch", patches, affine=3))
    assert rel_max_abs(got, merged) <= 1e-5


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("name,patches", [("ltx2_small", (1, 2)), ("ltx2_mid", (2, 3)),
                                          ("ltx2_tiny", (1, 2)), ("ltx2_tiny_n2", (1, 2))])
def test_ltx2_shaped_per_patch(v, name, patches, operands):
    got = host(gpu_decode(v, name, "patch", patches, operands=operands, launch="per_patch"))
    _bf16_bar(got, oracle_out(name, "whole"))


@pytest.mark.parametrize("operands", ["f16", "split"])
def test_ltx2_720p_one_frame_per_patch_every_value(v, operands):
    """The full-width 720p plan on one latent frame, each conv and GroupNorm launched per width
    quarter (10 latent columns and their halo, scaled at every stage): every output value."""
    got = host(gpu_decode(v, "ltx2_720p_1f", "patch", (1, 4), operands=operands,
                          launch="per_patch"))
    _bf16_bar(got, oracle_out("ltx2_720p_1f", "whole"))


def test_ltx2_720p_per_patch_against_golden(v):
    """The full 720p decode in four width quarters launched one by one, at the pixels the oracle's
    fp64 decode stored (seams of the quarters included)."""
    g = _golden("whole")
    _check_golden(g, gpu_decode(v, "ltx2_720p", "patch", (1, 4), launch="per_patch"))


@pytest.mark.parametrize("name,patches", [("mixed_rms_gn", (1, 2)), ("wan_tiny", (2, 2))])
def test_rms_plans_per_patch(v, name, patches):
    """Plans with RMS norms and the frame attention (one launch each) around per-patch convs, and
    a GroupNorm fed by an RMS block's second conv, per patch."""
    import torch
    spec = vae_synth.WORKLOADS[name]
    z = v.pad_latent(ndhwc(vae_synth.latent(spec)), spec)
    p = vae_synth.decoder_params(spec, affine_seed=5)
    dec = v.upload_decoder(spec, p)
    dec.set_launch(v.VAE_LAUNCH_PER_PATCH)
    desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=patches)
    ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
    out = torch.full(oracle.output_shape(spec, ndhwc(vae_synth.latent(spec)).shape),
                     float("nan"), device="cuda", dtype=torch.float32)
    dec.vae_decode_tiled(dev(z, "bf16"), desc, out, ws)
    torch.cuda.synchronize()
    dec.close()
    _bf16_bar(host(out), oracle.decode(spec, ndhwc(vae_synth.latent(spec)), p))


def test_per_patch_decode_is_deterministic(v):
    import torch
    a, b = gpu_decode(v, "ltx2_small", "patch", (1, 2), repeat=2, launch="per_patch")
    assert torch.equal(a, b)


def test_per_patch_timing_records(v):
    """Each per-patch launch is recorded with its patch index; the patches' conv work adds up to
    the whole decode's, and the statistics merges are recorded as shared work (-1)."""
    recs, merged = [], []
    gpu_decode(v, "ltx2_tiny", "patch", (1, 2), launch="per_patch", timing=recs)
    gpu_decode(v, "ltx2_tiny", "patch", (1, 2), timing=merged)
    conv = [r for r in recs if r["kind"] == "conv"]
    assert {r["tile"] for r in conv} == {0, 1}
    assert any(r["tile"] == -1 and r["kind"] == "gn" for r in recs)
    whole = sum(r["flops"] for r in merged if r["kind"] == "conv")
    assert abs(sum(r["flops"] for r in conv) - whole) <= 1e-9 * whole
    per = [sum(r["flops"] for r in conv if r["tile"] == t) for t in (0, 1)]
    assert per[0] == per[1]                        # two equal bands of 3 latent columns


# ------------------------------------------------------------------------------------------------
# The fp16 operand hand-off's range guards
# ------------------------------------------------------------------------------------------------

def test_f16_weight_pack_refuses_weights_past_the_scale(v):
    """fp16-packed weights are w * 2^10: a weight of magnitude 64 would overflow fp16 and is
    refused; 63.75 (65280 after the scale) packs, exactly; the bf16 packing takes both."""
    import torch
    w = torch.zeros((32, 3, 3, 3, 32), dtype=torch.bfloat16, device="cuda")
    w[3, 1, 2, 0, 7] = 63.75
    p = v.vae_conv_weight_pack_f16(w)
    torch.cuda.synchronize()
    assert float(p.view(torch.float16).abs().max()) == 63.75 * 1024
    w[5, 0, 0, 1, 9] = -64.0
    with pytest.raises(v.VaeError) as e:
        v.vae_conv_weight_pack_f16(w)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    v.vae_conv_weight_pack(w)                     # bf16 operands have no such limit
    w[5, 0, 0, 1, 9] = float("inf")
    with pytest.raises(v.VaeError):
        v.vae_conv_weight_pack_f16(w)


def test_decoder_pack_names_the_conv_past_the_fp16_range(v):
    """A large weight in a conv with fp16 operands (the first upsampling conv, conv 3 in plan
    order) is refused at packing with that conv's index; the same weight in conv_in (bf16
    operands) is accepted."""
    import copy
    params = copy.deepcopy(params_of("ltx2_tiny"))
    conv_params = [p for p in params if p["kind"] == "conv"]
    conv_params[0]["w"][0, 0, 0, 0, 0] = 100.0
    dec = v.upload_decoder(vae_synth.LTX2_TINY, params)   # packs: accepted
    dec.close()
    conv_params[3]["w"][1, 2, 1, 1, 0] = 100.0
    with pytest.raises(v.VaeError) as e:
        v.upload_decoder(vae_synth.LTX2_TINY, params)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["extent"] == 3


@pytest.mark.parametrize("name", ["ltx2_tiny", "wan_tiny"])
def test_decode_reports_activations_past_fp16(v, name):
    """A latent scaled by 1e6 drives the residual stream past 65504, where it is handed to an
    fp16-operand conv: the decode runs to the end (no fault), its output holds non-finite
    values, and vae_decode_status reports it. The unscaled decode reports nothing."""
    import torch
    spec = vae_synth.WORKLOADS[name]
    z = v.pad_latent(ndhwc(vae_synth.latent(spec)), spec)
    p = vae_synth.decoder_params(spec)
    dec = v.upload_decoder(spec, p)
    desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=(1, 2))
    ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
    out = torch.empty(oracle.output_shape(spec, ndhwc(vae_synth.latent(spec)).shape),
                      dtype=torch.float32, device="cuda")
    flags = []
    for scale in (1.0, 1e6, 1.0):
        dec.vae_decode_tiled(dev(z * scale, "bf16"), desc, out, ws)
        flags.append(dec.status(desc, ws))
        finite = bool(torch.isfinite(out).all())
        assert finite == (scale == 1.0), (scale, finite)
    dec.close()
    assert flags == [0, v.VAE_STATUS_NONFINITE, 0]
