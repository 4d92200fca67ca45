"""Pins of the oracle decoders: the patch-halo decode must equal the whole decode, a 1x1
overlap-blend grid must equal the whole decode, shapes follow the plan. No GPU."""
import numpy as np
import pytest

import oracle
import vae_synth


def ndhwc(a):
    return np.ascontiguousarray(np.asarray(a).transpose(0, 2, 3, 4, 1))


def _conv_gn_spec():
    s = vae_synth.CONV_GN
    return {"groups": s["groups"], "eps": s["eps"],
            "layers": [{"op": "conv", "cin": 32, "cout": 32}, {"op": "gn_silu"}]}


def _conv_gn_params(affine_seed=None):
    s = vae_synth.CONV_GN
    return [vae_synth.conv_params(0, s["cin"], s["cout"], "f32", affine_seed),
            vae_synth.gn_params(0, s["cout"], affine_seed)]


@pytest.mark.parametrize("affine", [None, 5])
def test_single_conv_gn_patches_equal_whole(affine):
    """Single conv + GN(8) + SiLU on [1,32,5,32,32], whole vs two width patches of 16 columns."""
    x = ndhwc(vae_synth.latent(vae_synth.CONV_GN))
    spec, params = _conv_gn_spec(), _conv_gn_params(affine)
    whole = oracle.decode(spec, x, params)
    split = oracle.decode_patch_halo(spec, x, params, (1, 2))
    assert whole.shape == (1, 5, 32, 32, 32)
    rel = np.abs(split - whole).max() / np.abs(whole).max()
    assert rel < 1e-12, rel


def test_tiny_decoder_shapes_and_patch_halo_equals_whole():
    spec = vae_synth.TINY_DECODER
    z = ndhwc(vae_synth.latent(spec))
    params = vae_synth.decoder_params(spec, affine_seed=3)
    whole = oracle.decode(spec, z, params)
    assert whole.shape == (1, 5, 64, 64, 3) == oracle.output_shape(spec, z.shape)
    for grid in [(2, 2), (1, 3), (3, 1)]:
        split = oracle.decode_patch_halo(spec, z, params, grid)
        rel = np.abs(split - whole).max() / np.abs(whole).max()
        assert rel < 1e-11, (grid, rel)


def test_overlap_blend_single_tile_is_whole_decode():
    spec = vae_synth.TINY_DECODER
    z = ndhwc(vae_synth.latent(spec))
    params = vae_synth.decoder_params(spec)
    whole = oracle.decode(spec, z, params)
    one = oracle.decode_overlap_blend(spec, z, params, (16, 16), (16, 16), spec["scale"])
    assert np.array_equal(one, whole)


def test_overlap_blend_differs_from_whole_only_by_tiling():
    """Mode B uses per-tile GroupNorm statistics and borders, so it must not equal the untiled
    decode; it is finite, has the right shape, and stays close in scale."""
    spec = vae_synth.TINY_DECODER
    z = ndhwc(vae_synth.latent(spec))
    params = vae_synth.decoder_params(spec)
    whole = oracle.decode(spec, z, params)
    tiled = oracle.decode_overlap_blend(spec, z, params, spec["overlap_tile"],
                                        spec["overlap_stride"], spec["scale"])
    assert tiled.shape == whole.shape and np.all(np.isfinite(tiled))
    diff = np.abs(tiled - whole).max()
    assert 1e-6 < diff < 10 * np.abs(whole).max()


def test_ltx2_small_patch_halo_equals_whole():
    spec = vae_synth.LTX2_SMALL
    z = ndhwc(vae_synth.latent(spec))
    params = vae_synth.decoder_params(spec)
    whole = oracle.decode(spec, z, params)
    assert whole.shape == oracle.output_shape(spec, z.shape) == (1, 9, 96, 160, 3)
    split = oracle.decode_patch_halo(spec, z, params, spec["patch_grid"])
    assert np.abs(split - whole).max() / np.abs(whole).max() < 1e-11


def test_720p_output_shape():
    spec = vae_synth.LTX2_720P
    assert oracle.output_shape(spec, (1, 16, 22, 40, 128)) == (1, 121, 704, 1280, 3)
    assert oracle.output_shape(vae_synth.LTX2_MID, (1, 3, 4, 6, 128)) == (1, 17, 128, 192, 3)


def _torch_decode(spec, z, params):
    """The same layer plan built from torch CPU library ops (float64, NCDHW)."""
    import torch
    import torch.nn.functional as F
    g, eps = spec["groups"], spec["eps"]
    it = iter(params)

    def conv(h, p):
        hp = F.pad(torch.cat([h[:, :, :1], h[:, :, :1], h], dim=2), (1, 1, 1, 1, 0, 0))
        return F.conv3d(hp, torch.from_numpy(p["w"]).double(), torch.from_numpy(p["b"]).double())

    def gn(h, p):
        return F.silu(F.group_norm(h, g, torch.from_numpy(p["gamma"]).double(),
                                   torch.from_numpy(p["beta"]).double(), eps))

    def rms(h, p):
        # torch's rms_norm normalises the trailing dims: move channels last, then back
        y = F.rms_norm(h.permute(0, 2, 3, 4, 1), (h.shape[1],),
                       torch.from_numpy(p["gamma"]).double(), eps)
        return (y + torch.from_numpy(p["beta"]).double()).permute(0, 4, 1, 2, 3)

    def attn(h, p):
        n, c, t, hh, ww = h.shape
        xn = rms(h, p).permute(0, 2, 3, 4, 1).reshape(n * t, 1, hh * ww, c)
        qkv = F.linear(xn, torch.from_numpy(p["w_qkv"]).double(),
                       torch.from_numpy(p["b_qkv"]).double())
        q, k, v = qkv.split(c, dim=-1)
        o = F.scaled_dot_product_attention(q, k, v)           # softmax(q k^T / sqrt(c)) v
        y = F.linear(o, torch.from_numpy(p["w_out"]).double(), torch.from_numpy(p["b_out"]).double())
        return y.reshape(n, t, hh, ww, c).permute(0, 4, 1, 2, 3) + h

    h = torch.from_numpy(z).double().permute(0, 4, 1, 2, 3)
    for op in spec["layers"]:
        k = op["op"]
        if k == "conv":
            h = conv(h, next(it))
        elif k == "res":
            g1, c1, g2, c2 = next(it), next(it), next(it), next(it)
            h = conv(gn(conv(gn(h, g1), c1), g2), c2) + h
        elif k == "res_rms":
            g1, c1, g2, c2 = next(it), next(it), next(it), next(it)
            h = conv(F.silu(rms(conv(F.silu(rms(h, g1)), c1), g2)), c2) + h
        elif k == "gn_silu":
            h = gn(h, next(it))
        elif k == "rms_silu":
            h = F.silu(rms(h, next(it)))
        elif k == "attn":
            h = attn(h, next(it))
        elif k == "conv_down":
            # two causal front copies of frame 0, the spatial zero pads, then a strided conv3d
            p = next(it)
            (pt, pb), (pl, pr) = {"around": ((1, 1), (1, 1)), "after": ((0, 1), (0, 1))}[op["pad"]]
            hp = F.pad(torch.cat([h[:, :, :1], h[:, :, :1], h], dim=2), (pl, pr, pt, pb, 0, 0))
            h = F.conv3d(hp, torch.from_numpy(p["w"]).double(), torch.from_numpy(p["b"]).double(),
                         stride=(op["st"], op["sh"], op["sw"]))
        elif k == "s2d":
            # causal front pad of st-1 copies of frame 0, then fold (dt, dh, dw) slowest into C
            st, sh, sw = op["st"], op["sh"], op["sw"]
            h = torch.cat([h[:, :, :1]] * (st - 1) + [h], dim=2)
            n, c, t, hh, ww = h.shape
            h = h.reshape(n, c, t // st, st, hh // sh, sh, ww // sw, sw)
            h = h.permute(0, 3, 5, 7, 1, 2, 4, 6).reshape(n, st * sh * sw * c, t // st,
                                                          hh // sh, ww // sw)
        elif k == "nearest":
            h = F.interpolate(h, scale_factor=(1, op["sh"], op["sw"]), mode="nearest")
        elif k == "d2s":
            st, sh, sw = op["st"], op["sh"], op["sw"]
            n, ck, t, hh, ww = h.shape
            c = ck // (st * sh * sw)
            h = h.reshape(n, st, sh, sw, c, t, hh, ww).permute(0, 4, 5, 1, 6, 2, 7, 3)
            h = h.reshape(n, c, t * st, hh * sh, ww * sw)[:, :, st - 1:]
    return h.permute(0, 2, 3, 4, 1).numpy()


def test_tiny_decoder_matches_torch_library_graph():
    spec = vae_synth.TINY_DECODER
    z = ndhwc(vae_synth.latent(spec))
    params = vae_synth.decoder_params(spec, affine_seed=7)
    ref = _torch_decode(spec, z, params)
    got = oracle.decode(spec, z, params)
    assert np.abs(got - ref).max() / np.abs(ref).max() < 1e-11


@pytest.mark.parametrize("name", ["wan_tiny", "ltx2_enc_tiny", "ltx2_enc_strided_tiny",
                                  "wan_enc_tiny"])
def test_plan_matches_torch_library_graph(name):
    """The RMS-norm residual blocks, the frame attention (torch's rms_norm, linear and
    scaled_dot_product_attention), the space-to-depth folds (a reshape) and the strided
    downsampling convs (torch's strided conv3d) of the Wan-shaped decoder and the LTX-2- and
    Wan-style encoders, rebuilt from torch CPU library ops, with random biases, gammas and
    betas."""
    spec = vae_synth.WORKLOADS[name]
    z = ndhwc(vae_synth.latent(spec)).astype(np.float64)
    params = vae_synth.decoder_params(spec, affine_seed=11)
    ref = _torch_decode(spec, z, params)
    got = oracle.decode(spec, z, params)
    assert got.shape == ref.shape == oracle.output_shape(spec, z.shape)
    assert np.abs(got - ref).max() / np.abs(ref).max() < 1e-11


def test_torch_library_graph_detects_a_planted_error():
    """Negative control: an oracle attention with its query projection's bias dropped must differ
    from the library graph by far more than the pin's tolerance. (A key bias would not do: it
    adds the same logit to every key of a query, which the softmax cancels.)"""
    spec = vae_synth.WAN_TINY
    z = ndhwc(vae_synth.latent(spec)).astype(np.float64)
    params = vae_synth.decoder_params(spec, affine_seed=11)
    ref = _torch_decode(spec, z, params)
    c = next(p for p in params if p["kind"] == "attn")["c"]
    bad = [dict(p) for p in params]
    for p in bad:
        if p["kind"] == "attn":
            p["b_qkv"] = np.asarray(p["b_qkv"]).copy()
            p["b_qkv"][:c] = 0.0
    got = oracle.decode(spec, z, bad)
    assert np.abs(got - ref).max() / np.abs(ref).max() > 1e-6


@pytest.mark.parametrize("name,grid", [("wan_tiny", (2, 2)), ("wan_small", (1, 2))])
def test_wan_shaped_patch_halo_equals_whole(name, grid):
    """RMS norms reduce over channels and the attention gathers whole frames, so the patch-halo
    decode of the Wan-shaped plan equals the whole decode."""
    spec = vae_synth.WORKLOADS[name]
    z = np.ascontiguousarray(vae_synth.latent(spec).transpose(0, 2, 3, 4, 1)).astype(np.float64)
    p = vae_synth.decoder_params(spec, affine_seed=7)
    whole = oracle.decode(spec, z, p)
    assert whole.shape == oracle.output_shape(spec, z.shape)
    patch = oracle.decode_patch_halo(spec, z, p, grid)
    assert np.abs(patch - whole).max() <= 1e-9 * np.abs(whole).max()


def test_wan_shaped_output_shape():
    spec = vae_synth.WAN_720P
    assert oracle.output_shape(spec, (1, 21, 44, 80, 48)) == (1, 81, 704, 1280, 3)


@pytest.mark.parametrize("name,clip", [("wan_tiny", 1), ("wan_tiny", 2), ("wan_small", 1)])
def test_causal_clips_equal_whole_decode(name, clip):
    """Clip by clip with each causal conv's last two input frames carried to the next clip: the
    whole decode, frame for frame."""
    spec = vae_synth.WORKLOADS[name]
    z = ndhwc(vae_synth.latent(spec)).astype(np.float64)
    p = vae_synth.decoder_params(spec, affine_seed=6)
    whole = oracle.decode(spec, z, p)
    clips = oracle.decode_causal_clips(spec, z, p, clip)
    assert clips.shape == whole.shape
    assert np.abs(clips - whole).max() <= 1e-12 * np.abs(whole).max()


def test_causal_clips_carry_information_across_the_boundary():
    """The carried frames matter: changing the last latent frame of the first clip changes the
    second clip's output (through the carry), and changing the second clip's first frame leaves
    every output frame of the first clip as it was (causality)."""
    spec = vae_synth.WAN_TINY
    z = ndhwc(vae_synth.latent(spec)).astype(np.float64)
    p = vae_synth.decoder_params(spec, affine_seed=6)
    base = oracle.decode_causal_clips(spec, z, p, 2)
    first = 1 + (2 - 1) * 4                       # output frames of latent frames [0, 2)
    z1 = z.copy()
    z1[:, 1] += 0.5
    a = oracle.decode_causal_clips(spec, z1, p, 2)
    assert np.abs(a[:, first:] - base[:, first:]).max() > 1e-3
    z2 = z.copy()
    z2[:, 2] += 0.5
    b = oracle.decode_causal_clips(spec, z2, p, 2)
    assert np.array_equal(b[:, :first], base[:, :first])
    assert np.abs(b[:, first:] - base[:, first:]).max() > 1e-3


def test_causal_clips_refuse_groupnorm_plans():
    """A GroupNorm's statistics span every frame: no clip-by-clip decode can reproduce it."""
    spec = vae_synth.LTX2_TINY
    z = ndhwc(vae_synth.latent(spec))
    with pytest.raises(AssertionError):
        oracle.decode_causal_clips(spec, z, vae_synth.decoder_params(spec), 1)


def test_first_frames_of_a_time_local_plan_depend_on_the_first_latent_frames():
    """For a plan whose every op is local in time (causal convs, RMS norms, per-frame attention,
    causal upsamplers: the Wan-shaped plan), the first 1 + (k - 1) * 4 output frames of a decode
    are the decode of the first k latent frames alone; the GPU's full-T Wan test relies on this.
    A GroupNorm plan is the control: its statistics span every frame, so the same frames differ."""
    spec = vae_synth.WAN_TINY
    z = ndhwc(vae_synth.latent(spec))
    p = vae_synth.decoder_params(spec, affine_seed=5)
    full = oracle.decode(spec, z, p)
    first = oracle.decode(vae_synth.with_latent(spec, (1, 48, 2, 4, 6), "wan_tiny_2f"), z[:, :2], p)
    assert first.shape[1] == 5
    np.testing.assert_allclose(full[:, :5], first, rtol=0, atol=1e-12 * np.abs(full).max())
    gspec = vae_synth.LTX2_MID
    gz = ndhwc(vae_synth.latent(gspec))
    gp = vae_synth.decoder_params(gspec)
    gfull = oracle.decode(gspec, gz, gp)
    gfirst = oracle.decode(vae_synth.with_latent(gspec, (1, 128, 2, 4, 6), "ltx2_mid_2f"),
                           gz[:, :2], gp)
    n = gfirst.shape[1]
    assert np.abs(gfull[:, :n] - gfirst).max() > 1e-3 * np.abs(gfull).max()
