"""Pins of the oracle's encode path: the space-to-depth fold, the encoder plan's shapes, and the
tiled encodes against the untiled one. No GPU."""
import itertools

import numpy as np
import pytest

import oracle
import vae_synth
from _util import ndhwc


@pytest.mark.parametrize("fold,t", [((2, 2, 2), 5), ((1, 4, 4), 3), ((2, 1, 3), 7), ((4, 2, 1), 9),
                                    ((1, 1, 1), 2)])
def test_space_to_depth_by_brute_force(fold, t):
    """Every output value against the definition, by explicit index loops: input frame
    st*t' + dt - (st - 1), clamped at 0 (the causal front copies of frame 0), row sh*h' + dh,
    column sw*w' + dw, into channel ((dt*sh + dh)*sw + dw)*C + c."""
    st, sh, sw = fold
    c = 3
    x = np.random.default_rng(7).standard_normal((1, t, 2 * sh, 3 * sw, c))
    y = oracle.space_to_depth(x, st, sh, sw)
    to = (t + st - 1) // st
    assert y.shape == (1, to, 2, 3, st * sh * sw * c)
    for tt, hh, ww, dt, dh, dw, cc in itertools.product(range(to), range(2), range(3), range(st),
                                                        range(sh), range(sw), range(c)):
        src = max(st * tt + dt - (st - 1), 0)
        ch = ((dt * sh + dh) * sw + dw) * c + cc
        assert y[0, tt, hh, ww, ch] == x[0, src, sh * hh + dh, sw * ww + dw, cc]


@pytest.mark.parametrize("fold,t", [((2, 2, 2), 9), ((1, 4, 4), 4), ((2, 1, 3), 3), ((4, 2, 2), 5)])
def test_depth_to_space_inverts_space_to_depth(fold, t):
    x = np.random.default_rng(8).standard_normal((2, t, 2 * fold[1], 3 * fold[2], 5))
    y = oracle.space_to_depth(x, *fold)
    assert np.array_equal(oracle.depth_to_space(y, *fold), x)


def test_encoder_plan_shapes():
    spec = vae_synth.LTX2_ENC_720P
    assert oracle.output_shape(spec, (1, 121, 704, 1280, 3)) == (1, 16, 22, 40, 256)
    assert oracle.output_shape(vae_synth.LTX2_ENC_SMALL, (1, 9, 64, 160, 3)) == (1, 2, 2, 5, 256)
    # the widths the configuration states: 128 / 256 / 512 / 1024
    widths = [op["c"] for op in spec["layers"] if op["op"] == "res"]
    assert sorted(set(widths)) == [128, 256, 512, 1024]


def _enc(name):
    spec = vae_synth.WORKLOADS[name]
    return spec, ndhwc(vae_synth.latent(spec)), vae_synth.decoder_params(spec, affine_seed=9)


def test_video_input_is_uniform_and_bf16_exact():
    spec, x, _ = _enc("ltx2_enc_small")
    assert x.min() >= -1.0 and x.max() <= 1.0 and x.std() > 0.5
    assert np.array_equal(vae_synth.round_bf16(x.astype(np.float32)), x.astype(np.float32))


def test_encode_patch_halo_equals_whole():
    """Bands in whole multiples of the 32-pixel fold (64 -> 32 + 32; 160 -> 96 + 64), halos read
    from the neighbours, GroupNorm statistics merged across patches: the untiled encode."""
    spec, x, p = _enc("ltx2_enc_small")
    whole = oracle.encode(spec, x, p)
    split = oracle.encode_patch_halo(spec, x, p, (2, 2))
    assert split.shape == whole.shape == (1, 2, 2, 5, 256)
    assert np.abs(split - whole).max() / np.abs(whole).max() < 1e-11


def test_encode_patch_halo_refuses_bands_off_the_fold():
    spec, x, p = _enc("ltx2_enc_small")
    with pytest.raises(AssertionError):
        oracle.decode_patch_halo(spec, x[:, :, :, :150], p, (1, 2), unit=(32, 32))


def test_encode_overlap_single_tile_is_whole():
    spec, x, p = _enc("ltx2_enc_tiny")
    whole = oracle.encode(spec, x, p)
    one = oracle.encode_overlap_blend(spec, x, p, (8, 8), (8, 8))
    assert np.array_equal(one, whole)


_FOLDS_ONLY = {
    # no convolution and no norm: every latent value depends on its own pixel block only
    "groups": 1, "eps": 1e-6, "down": (4, 8, 8),
    "layers": [{"op": "s2d", "st": 1, "sh": 4, "sw": 4},
               {"op": "s2d", "st": 2, "sh": 2, "sw": 1},
               {"op": "s2d", "st": 2, "sh": 1, "sw": 2}],
}


@pytest.mark.parametrize("tile,stride", [((2, 3), (1, 2)), ((3, 2), (2, 1)), ((1, 1), (1, 1))])
def test_encode_overlap_of_a_local_plan_is_the_whole_encode(tile, stride):
    """A plan of folds only pins the tile geometry: pixel crop [h0*32, h1*32) <-> latent rows
    [h0, h1), and the latent-space blend of identical overlaps."""
    x = np.random.default_rng(5).uniform(-1, 1, (1, 5, 4 * 8, 5 * 8, 3))
    whole = oracle.encode(_FOLDS_ONLY, x, [])
    assert whole.shape == (1, 2, 4, 5, 3 * 16 * 4 * 4)      # 5 frames -> 3 -> 2
    tiled = oracle.encode_overlap_blend(_FOLDS_ONLY, x, [], tile, stride)
    np.testing.assert_allclose(tiled, whole, rtol=1e-14, atol=1e-14)


def test_encode_overlap_blend_differs_from_whole_only_by_tiling():
    spec, x, p = _enc("ltx2_enc_small")
    whole = oracle.encode(spec, x, p)
    tiled = oracle.encode_overlap_blend(spec, x, p, spec["overlap_tile"], spec["overlap_stride"])
    assert tiled.shape == whole.shape and np.all(np.isfinite(tiled))
    assert 1e-6 < np.abs(tiled - whole).max() < 10 * np.abs(whole).max()


# ------------------------------------------------------------------------------------------------
# The bare strided downsampler conv and the encoders built on it
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("stride,pad,t", [((2, 2, 2), ((1, 1), (1, 1)), 5),   # LTX-2 kind
                                          ((1, 2, 2), ((0, 1), (0, 1)), 3),   # Wan: pad, stride
                                          ((2, 1, 2), ((1, 1), (0, 1)), 4)])
def test_strided_causal_conv_against_torch(stride, pad, t):
    """Against torch's own strided conv3d (CPU, float64) on the causally padded input."""
    import torch
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, t, 6, 8, 3))
    w = rng.standard_normal((4, 3, 3, 3, 3))
    b = rng.standard_normal(4)
    got = oracle.strided_causal_conv3d(x, w, b, stride, pad)
    xp = np.concatenate([x[:, :1]] * 2 + [x], axis=1)                 # causal front copies
    xt = torch.from_numpy(np.ascontiguousarray(xp.transpose(0, 4, 1, 2, 3)))
    xt = torch.nn.functional.pad(xt, (pad[1][0], pad[1][1], pad[0][0], pad[0][1], 0, 0))
    ref = torch.nn.functional.conv3d(xt, torch.from_numpy(w), torch.from_numpy(b), stride=stride)
    ref = ref.numpy().transpose(0, 2, 3, 4, 1)
    assert got.shape == ref.shape
    assert got.shape[1] == (t - 1) // stride[0] + 1
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_strided_causal_conv_by_brute_force():
    """Every output by explicit loops: frame st*t + a - 2 clamped at 0, row sh*h + p - top,
    column sw*w + q - left, zeros outside the image."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1, 3, 4, 5, 2))
    w = rng.standard_normal((2, 2, 3, 3, 3))
    stride, pad = (2, 2, 2), ((1, 1), (1, 1))
    y = oracle.strided_causal_conv3d(x, w, None, stride, pad)
    assert y.shape == (1, 2, 2, 3, 2)
    for t, h, ww, o in itertools.product(range(2), range(2), range(3), range(2)):
        acc = 0.0
        for c, a, p, q in itertools.product(range(2), range(3), range(3), range(3)):
            ti = max(2 * t + a - 2, 0)
            hi, wi = 2 * h + p - 1, 2 * ww + q - 1
            if 0 <= hi < 4 and 0 <= wi < 5:
                acc += w[o, c, a, p, q] * x[0, ti, hi, wi, c]
        assert abs(y[0, t, h, ww, o] - acc) < 1e-12


@pytest.mark.parametrize("name", ["ltx2_enc_strided_tiny", "wan_enc_tiny"])
def test_strided_encoder_patch_halo_equals_whole(name):
    """Patch bands in whole multiples of the plan's fold: each strided conv gathers its halo rows
    (one before the band for padding around, one after for padding after) from the neighbours
    and must reproduce the whole encode."""
    spec = vae_synth.WORKLOADS[name]
    x = np.ascontiguousarray(vae_synth.latent(spec).transpose(0, 2, 3, 4, 1)).astype(np.float64)
    p = vae_synth.decoder_params(spec, affine_seed=4)
    whole = oracle.encode(spec, x, p)
    assert whole.shape == oracle.output_shape(spec, x.shape)
    split = oracle.encode_patch_halo(spec, x, p, spec["patch_grid"])
    assert np.abs(split - whole).max() <= 1e-12 * np.abs(whole).max()


def test_strided_encoder_720p_shapes():
    """Three stride-2 downsamplers after the 4x4 patchify: [1,3,121,704,1280] ->
    [1,256,16,22,40], the frames 121 -> 61 -> 31 -> 16 by the causal rule."""
    spec = vae_synth.LTX2_ENC_STRIDED_720P
    assert oracle.output_shape(spec, (1, 121, 704, 1280, 3)) == (1, 16, 22, 40, 256)
    ts = [121]
    for op in spec["layers"]:
        if op["op"] == "conv_down":
            ts.append((ts[-1] - 1) // op["st"] + 1)
    assert ts == [121, 61, 31, 16]
