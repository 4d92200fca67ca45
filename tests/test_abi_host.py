"""Host-side tests of the C-ABI library: exported symbols, the tile split against the oracle
(bit-exact integers), and refusals. No GPU: only host code of the library runs."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def v():
    import video_diffusion_vae_amd as v
    return v


def header_symbols():
    with open(os.path.join(ROOT, "include", "vae.h")) as f:
        text = f.read()
    return set(re.findall(r"VAE_API\s+[\w\s\*]+?\b(vae_\w+)\s*\(", text))


def test_library_exports_every_header_symbol(v):
    names = header_symbols()
    assert len(names) >= 19
    lib = ctypes.CDLL(v._binding.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert names == set(v.EXPORTS)


def _fields(t):
    return {"latent": (t.latent.t0, t.latent.t1, t.latent.h0, t.latent.h1, t.latent.w0,
                       t.latent.w1),
            "out": (t.out.t0, t.out.t1, t.out.h0, t.out.h1, t.out.w0, t.out.w1),
            "lead": (t.lead_t, t.lead_h, t.lead_w), "trail": (t.trail_t, t.trail_h, t.trail_w),
            "row": t.row, "col": t.col}


PATCH_CASES = [
    (16, 22, 40, 1, 4, (8, 32, 32)), (3, 16, 16, 2, 2, (2, 4, 4)), (5, 17, 23, 3, 4, (1, 1, 1)),
    (1, 7, 7, 7, 7, (8, 32, 32)), (9, 22, 40, 4, 4, (2, 8, 8)), (13, 5, 11, 1, 3, (4, 2, 2)),
]

OVERLAP_CASES = [
    (16, 22, 40, (16, 16), (14, 14), (8, 32, 32)), (1, 576, 576, (512, 512), (448, 448), (1, 1, 1)),
    (1, 256, 256, (512, 512), (448, 448), (1, 1, 1)), (3, 16, 16, (8, 8), (6, 6), (2, 4, 4)),
    (5, 30, 17, (16, 5), (14, 2), (2, 3, 5)), (2, 9, 9, (4, 9), (4, 3), (1, 8, 8)),
    (9, 13, 29, (7, 6), (7, 1), (1, 4, 4)), (1, 1, 1, (1, 1), (1, 1), (1, 1, 1)),
]

# with temporal tiles: (T, H, W, tile_hw, stride_hw, scale, tile_t, stride_t)
TEMPORAL_CASES = [
    (16, 22, 40, (16, 16), (14, 14), (8, 32, 32), 8, 6),      # 3 clips, 9 shared output frames
    (16, 22, 40, (0, 0), (0, 0), (8, 32, 32), 4, 1),          # contained clips at the end
    (15, 44, 80, (32, 32), (28, 28), (4, 16, 16), 8, 7),      # a one-frame last clip [14, 15)
    (7, 9, 8, (5, 4), (3, 3), (4, 2, 2), 3, 2),
    (16, 4, 4, (0, 0), (0, 0), (1, 1, 1), 8, 8),              # scale 1: abutting clips allowed
    (3, 16, 16, (8, 8), (6, 6), (2, 4, 4), 2, 1),
    (5, 3, 3, (0, 0), (0, 0), (2, 1, 1), 9, 1),               # tile longer than T: T whole
]


@pytest.mark.parametrize("case", PATCH_CASES)
def test_patch_split_bit_exact(v, case):
    t, h, w, ph, pw, scale = case
    got = v.vae_tile_split(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (2, t, h, w, 8), scale,
                                         patches=(ph, pw)))
    ref = oracle.patch_tiles(t, h, w, ph, pw, scale)
    assert len(got) == len(ref)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert g.index == i
        f = _fields(g)
        assert f["latent"] == r["latent"] and f["out"] == r["out"]
        assert f["lead"] == r["lead"] and f["trail"] == r["trail"]
        assert (f["row"], f["col"]) == (r["row"], r["col"])


@pytest.mark.parametrize("case", OVERLAP_CASES)
def test_overlap_split_bit_exact(v, case):
    t, h, w, tile, stride, scale = case
    got = v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, t, h, w, 8), scale,
                                         tile=tile, stride=stride))
    ref = oracle.overlap_tiles(t, h, w, tile, stride, scale)
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        f = _fields(g)
        for k in ("latent", "out", "lead", "trail"):
            assert f[k] == r[k], (k, f[k], r[k])


@pytest.mark.parametrize("case", TEMPORAL_CASES)
def test_temporal_overlap_split_bit_exact(v, case):
    t, h, w, tile, stride, scale, tt, stt = case
    got = v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, t, h, w, 8), scale,
                                         tile=tile, stride=stride, tile_t=tt, stride_t=stt))
    ref = oracle.overlap_tiles(t, h, w, tile, stride, scale, tt, stt)
    assert len(got) == len(ref)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert g.index == i
        f = _fields(g)
        for k in ("latent", "out", "lead", "trail", "row", "col"):
            assert f[k] == r[k], (k, f[k], r[k])


def test_temporal_gap_is_refused_with_numbers(v):
    with pytest.raises(v.VaeError) as e:
        v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, 16, 4, 4, 8), (8, 1, 1),
                                       tile_t=8, stride_t=8))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    assert e.value.info["axis"] == 1 and e.value.info["extent"] == 8
    with pytest.raises(v.VaeError) as e:
        v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, 16, 4, 4, 8), (1, 1, 1),
                                       tile_t=4, stride_t=5))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 1


def test_refusals_carry_numbers(v):
    with pytest.raises(v.VaeError) as e:
        v.vae_tile_split(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 4, 3, 40, 8), (1, 1, 1),
                                       patches=(4, 1)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    assert e.value.info["axis"] == 2 and e.value.info["extent"] == 3
    assert e.value.info["min_width"] == 4
    with pytest.raises(v.VaeError) as e:
        v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, 4, 40, 40, 8), (1, 1, 1),
                                       tile=(8, 8), stride=(9, 8)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 2
    with pytest.raises(v.VaeError) as e:
        v.vae_tile_split(v.tiling_desc(7, (1, 4, 40, 40, 8), (1, 1, 1)))
    assert e.value.status == v.VAE_ERR_INVALID_ARG


def test_decoder_plan_validation(v):
    import vae_synth
    spec = vae_synth.TINY_DECODER
    fake = [None] * 100
    with pytest.raises(v.VaeError) as e:      # wrong pointer count
        v.Decoder(v.VAE_DTYPE_F32, 16, 32, 1e-6, spec["layers"], fake[:3])
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    bad = [dict(op) for op in spec["layers"]]
    bad[0] = {"op": "conv", "cin": 8, "cout": 128}
    with pytest.raises(v.VaeError):           # channels do not chain
        v.Decoder(v.VAE_DTYPE_F32, 16, 32, 1e-6, bad, fake[:0])
    with pytest.raises(v.VaeError) as e:      # bf16 activation storage misses the bf16 bar
        v.Decoder(v.VAE_DTYPE_BF16, 16, 32, 1e-6, spec["layers"], fake[:0],
                  act_dtype=v.VAE_DTYPE_BF16)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    assert "fp32" in str(e.value)
    with pytest.raises(v.VaeError) as e:      # an fp32 plan cannot store bf16 activations
        v.Decoder(v.VAE_DTYPE_F32, 16, 32, 1e-6, spec["layers"], fake[:0],
                  act_dtype=v.VAE_DTYPE_BF16)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    with pytest.raises(v.VaeError) as e:      # split and fp16 operands together
        v.Decoder(v.VAE_DTYPE_BF16, 16, 32, 1e-6, spec["layers"], fake[:0],
                  flags=v.VAE_DECODE_SPLIT_FP32_OPERANDS | v.VAE_DECODE_F16_OPERANDS)
    assert e.value.status == v.VAE_ERR_INVALID_ARG


def test_workspace_query_needs_no_gpu(v):
    import vae_synth
    spec = vae_synth.LTX2_720P
    n_ptr = sum({"conv": 2, "res": 8, "gn_silu": 2}.get(op["op"], 0) for op in spec["layers"])
    # dummy non-null, 16-byte aligned pointers: creating a decoder never dereferences them
    ptrs = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(n_ptr)]

    class P:
        def __init__(self, p):
            self.p = p

        def data_ptr(self):
            return self.p.value
    dec = v.Decoder(v.VAE_DTYPE_BF16, 128, 32, 1e-6, spec["layers"], [P(p) for p in ptrs],
                    flags=v.VAE_DECODE_F16_OPERANDS)
    a = dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 16, 22, 40, 128),
                                         (8, 32, 32), patches=(1, 4)))
    b = dec.workspace_size(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, 16, 22, 40, 128),
                                         (8, 32, 32), tile=(16, 16), stride=(14, 14)))
    # three rotating buffers of the largest activation (the 1024-channel S2 conv output, bf16)
    assert a >= 3 * 858880 * 1024 * 2
    assert b < a                                  # tiles are smaller than the whole tensor
    with pytest.raises(v.VaeError) as e:          # more patches than the decoder's 16
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 16, 22, 40, 128),
                                         (8, 32, 32), patches=(5, 4)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    with pytest.raises(v.VaeError):               # scales that do not match the plan
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 16, 22, 40, 128),
                                         (8, 16, 32), patches=(1, 4)))
    # per-patch launches keep every patch box's GroupNorm slots and moments: never smaller
    dec.set_launch(v.VAE_LAUNCH_PER_PATCH)
    c = dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 16, 22, 40, 128),
                                         (8, 32, 32), patches=(1, 4)))
    assert c >= a
    # the overlap-blend mode decodes one tile at a time and ignores the setting
    assert dec.workspace_size(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, 16, 22, 40, 128),
                                            (8, 32, 32), tile=(16, 16), stride=(14, 14))) == b
    with pytest.raises(v.VaeError) as e:
        dec.set_launch(2)
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    dec.close()


class _FakePtr:
    """A non-null device-pointer stand-in: creating a decoder never dereferences it."""

    def __init__(self, i):
        self.p = 0x1000 * (i + 1)

    def data_ptr(self):
        return self.p


def _mixed_plan(block):
    return [{"op": "conv", "cin": 32, "cout": 128}, {"op": block, "c": 128}, {"op": "gn_silu"},
            {"op": "conv", "cin": 128, "cout": 32, "f32_out": True}]


@pytest.mark.parametrize("flags", ["f16", "none"])
def test_mixed_rms_gn_plan_workspace_holds_fused_partials(v, flags):
    """The second conv of a RES_RMS block gathers the statistics of a GroupNorm that follows it in
    its epilogue: the decode workspace must hold those partials. Sized like a RES block's (whose
    first conv gathers partials of the same shape), and at least three activation buffers plus
    the partials that vae_conv3d_causal_fused_workspace reports for that conv."""
    import torch
    shape = (1, 5, 64, 64, 32)
    fl = v.VAE_DECODE_F16_OPERANDS if flags == "f16" else 0
    sizes = {}
    for block in ("res", "res_rms"):
        layers = _mixed_plan(block)
        n_ptr = sum({"conv": 2, "res": 8, "res_rms": 8, "gn_silu": 2}[op["op"]] for op in layers)
        dec = v.Decoder(v.VAE_DTYPE_BF16, 32, 32, 1e-6, layers,
                        [_FakePtr(i) for i in range(n_ptr)], flags=fl)
        sizes[block] = dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, shape, (1, 1, 1)))
        dec.close()
    x = torch.zeros((1, 5, 64, 64, 128), dtype=torch.bfloat16)
    w = torch.zeros((128, 3, 3, 3, 128), dtype=torch.bfloat16)
    y = torch.zeros((1, 5, 64, 64, 128), dtype=torch.float32)
    part = v.vae_conv3d_causal_fused_workspace(x, w, y, gn_groups=32)
    assert part > 0
    act = 5 * 64 * 64 * 128 * 4                   # the largest activation: fp32, 128 channels
    assert sizes["res_rms"] >= 3 * act + part
    assert sizes["res_rms"] == sizes["res"]


@pytest.mark.parametrize("case", [((121, 704, 1280), (16, 16), (14, 14)),
                                  ((9, 64, 160), (2, 3), (2, 2)),
                                  ((9, 64, 96), (2, 2), (1, 1))])
def test_encoder_overlap_split_on_the_latent_grid(v, case):
    """An encoder desc (down = 8, 32, 32) cuts its tiles on the latent grid: `out` is the latent
    box (all latent frames), `latent` the input-video box (rows and columns times 32, all input
    frames); overlaps are latent samples."""
    (t, h, w), tile, stride = case
    lt, lh, lw = (t + 7) // 8, h // 32, w // 32
    got = v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, t, h, w, 4), (1, 1, 1),
                                         tile=tile, stride=stride, down=(8, 32, 32)))
    ref = oracle.overlap_tiles(lt, lh, lw, tile, stride, (1, 1, 1))
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        f = _fields(g)
        assert f["out"] == r["out"] == r["latent"]
        _, _, h0, h1, w0, w1 = r["latent"]
        assert f["latent"] == (0, t, 32 * h0, 32 * h1, 32 * w0, 32 * w1)
        assert f["lead"] == r["lead"] and f["trail"] == r["trail"]


def test_encoder_patch_split_in_fold_units(v):
    """Patch-halo bands of an encoder are whole multiples of its fold (the band rule over latent
    rows): 2 latent rows -> 1 + 1, 5 latent columns -> 3 + 2; `latent` holds the pixel box."""
    got = v.vae_tile_split(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 9, 64, 160, 4), (1, 1, 1),
                                         patches=(2, 2), down=(8, 32, 32)))
    ref = oracle.patch_tiles(2, 2, 5, 2, 2, (1, 1, 1))
    assert len(got) == len(ref) == 4
    for g, r in zip(got, ref):
        f = _fields(g)
        assert f["out"] == r["latent"]
        _, _, h0, h1, w0, w1 = r["latent"]
        assert f["latent"] == (0, 9, 32 * h0, 32 * h1, 32 * w0, 32 * w1)
    with pytest.raises(v.VaeError) as e:          # 3 latent columns cannot take 4 bands
        v.vae_tile_split(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 9, 64, 96, 4), (1, 1, 1),
                                       patches=(1, 4), down=(8, 32, 32)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 3


def test_encoder_tiling_refusals(v):
    with pytest.raises(v.VaeError) as e:          # temporal tiles with folds
        v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, 9, 64, 96, 4), (1, 1, 1),
                                       tile=(2, 2), stride=(1, 1), tile_t=2, stride_t=1,
                                       down=(8, 32, 32)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    with pytest.raises(v.VaeError) as e:          # 100 rows do not fold by 32
        v.vae_tile_split(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, 9, 100, 96, 4), (1, 1, 1),
                                       tile=(2, 2), stride=(1, 1), down=(8, 32, 32)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 2


def test_encoder_plan_tilings(v):
    """An encoder plan (space-to-depth folds) takes the 4-channel padded video, sizes its
    workspace untiled, in fold-unit patches and in latent-grid overlap tiles, and refuses tilings
    without the plan's folds and extents its folds do not divide."""
    import vae_synth
    spec = vae_synth.LTX2_ENC_720P
    assert v.latent_channels(spec) == 4                # 3 -> 4: the 4x4 patchify gives 64
    layers = [dict(op) for op in spec["layers"]]
    layers[1]["cin"] = 64
    n_ptr = sum({"conv": 2, "res": 8, "gn_silu": 2}.get(op["op"], 0) for op in layers)
    ptrs = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(n_ptr)]

    class P:
        def __init__(self, p):
            self.p = p

        def data_ptr(self):
            return self.p.value
    dec = v.Decoder(v.VAE_DTYPE_BF16, 4, 32, 1e-6, layers, [P(p) for p in ptrs],
                    flags=v.VAE_DECODE_F16_OPERANDS)
    shape = (1, 121, 704, 1280, 4)
    a = dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, shape, (1, 1, 1)))
    # the largest activation: the 128-channel fp32 stage-0 tensor, 121 x 176 x 320
    assert a >= 3 * 121 * 176 * 320 * 128 * 4
    with pytest.raises(v.VaeError) as e:          # patches need the plan's folds in down
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, shape, (1, 1, 1),
                                         patches=(1, 2)))
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    c = dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, shape, (1, 1, 1),
                                         patches=(1, 4), down=(8, 32, 32)))
    assert c >= a
    with pytest.raises(v.VaeError) as e:          # overlap tiles need the plan's folds in down
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, shape, (1, 1, 1),
                                         tile=(16, 16), stride=(14, 14)))
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    with pytest.raises(v.VaeError) as e:          # folds that are not the plan's
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, shape, (1, 1, 1),
                                         tile=(16, 16), stride=(14, 14), down=(8, 16, 16)))
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    b = dec.workspace_size(v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, shape, (1, 1, 1),
                                         tile=(16, 16), stride=(14, 14), down=(8, 32, 32)))
    assert 0 < b < a                              # a 512 x 512 pixel tile at a time
    with pytest.raises(v.VaeError) as e:          # 120 frames do not fold causally by 2
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 120, 704, 1280, 4),
                                         (1, 1, 1)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 1
    with pytest.raises(v.VaeError) as e:          # 700 rows do not fold by 4 then 2, 2, 2
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 121, 700, 1280, 4),
                                         (1, 1, 1)))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 2
    dec.close()


def test_fused_conv_validation_needs_no_gpu(v):
    """Argument checks and the workspace query of vae_conv3d_causal_fused run on the host only
    (host tensors stand in for device buffers; nothing is launched)."""
    import torch
    x = torch.zeros((1, 2, 4, 8, 64), dtype=torch.bfloat16)
    w = torch.zeros((256, 3, 3, 3, 64), dtype=torch.bfloat16)
    y = torch.zeros((1, 3, 8, 16, 32), dtype=torch.float32)   # d2s (2, 2, 2): 2T-1, 2H, 2W
    # one 256-position block, eight sub-positions, one wave row: 8 slots per (sample, group)
    n = v.vae_conv3d_causal_fused_workspace(x, w, y, d2s=(2, 2, 2), gn_groups=8)
    assert n == 1 * 8 * 8 * 3 * 8
    assert v.vae_conv3d_causal_fused_workspace(x, w, y, d2s=(2, 2, 2)) == 0
    with pytest.raises(v.VaeError) as e:          # y does not match the factors
        v.vae_conv3d_causal_fused_workspace(x, w, y, d2s=(1, 2, 2))
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    with pytest.raises(v.VaeError) as e:          # a fused depth-to-space needs the MFMA path
        x16 = torch.zeros((1, 2, 4, 8, 16), dtype=torch.bfloat16)
        v.vae_conv3d_causal_fused_workspace(x16, w[..., :16], y, d2s=(2, 2, 2))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    with pytest.raises(v.VaeError) as e:          # groups must divide the channels
        v.vae_conv3d_causal_fused_workspace(x, w, y, d2s=(2, 2, 2), gn_groups=5)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    # a nearest upsampling of x read by the conv: y follows the upsampled grid
    yu = torch.zeros((1, 3, 16, 32, 32), dtype=torch.float32)   # d2s (2,2,2) of an 8x16 grid
    assert v.vae_conv3d_causal_fused_workspace(x, w, yu, d2s=(2, 2, 2), in_up=(2, 2)) == 0
    with pytest.raises(v.VaeError) as e:          # y does not follow the upsampled grid
        v.vae_conv3d_causal_fused_workspace(x, w, y, d2s=(2, 2, 2), in_up=(2, 2))
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    with pytest.raises(v.VaeError) as e:          # factors must be powers of two
        v.vae_conv3d_causal_fused_workspace(x, w, y, d2s=(2, 2, 2), in_up=(3, 1))
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    # an input GroupNorm: fp32 (or fp16 with bf16-packed weights), packed weights, no fp32 split
    xf = torch.zeros((1, 2, 4, 8, 64), dtype=torch.float32)
    xh = torch.zeros((1, 2, 4, 8, 64), dtype=torch.float16)
    ab = torch.zeros((1, 64, 2), dtype=torch.float32)
    P, PH = v.VAE_CONV_PACKED_WEIGHTS, v.VAE_CONV_PACKED_F16_WEIGHTS
    for xx, fl in ((xf, P), (xf, PH), (xh, P)):
        assert v.vae_conv3d_causal_fused_workspace(xx, w, y, d2s=(2, 2, 2), flags=fl,
                                                   in_scale_shift=ab) == 0
    for xx, fl, status in ((xf, 0, v.VAE_ERR_UNSUPPORTED),                 # standard weights
                           (xf, P | v.VAE_CONV_SPLIT_FP32, v.VAE_ERR_UNSUPPORTED),
                           (x, P, v.VAE_ERR_UNSUPPORTED),                  # bf16 x
                           (xh, PH, v.VAE_ERR_UNSUPPORTED)):               # fp16 x, fp16 weights
        with pytest.raises(v.VaeError) as e:
            v.vae_conv3d_causal_fused_workspace(xx, w, y, d2s=(2, 2, 2), flags=fl,
                                                in_scale_shift=ab)
        assert e.value.status == status, (xx.dtype, fl)
    with pytest.raises(v.VaeError) as e:          # the scale and shift must be 16-byte aligned
        v.vae_conv3d_causal_fused_workspace(xf, w, y, d2s=(2, 2, 2), flags=P,
                                            in_scale_shift=ab.view(-1)[1:])
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    # vae_groupnorm_scale_shift refuses before launching: channels not a multiple of groups, a
    # misaligned output
    mr = ctypes.c_void_p(1 << 40)
    assert v.LIB.vae_groupnorm_scale_shift(mr, 1, 60, 8, None, None, ctypes.c_void_p(1 << 41),
                                           None) == v.VAE_ERR_INVALID_ARG
    assert v.LIB.vae_groupnorm_scale_shift(mr, 1, 64, 8, None, None,
                                           ctypes.c_void_p((1 << 41) + 4),
                                           None) == v.VAE_ERR_INVALID_ARG


def test_space_to_depth_validation_needs_no_gpu(v):
    """vae_space_to_depth's argument checks run on the host (host tensors stand in for device
    buffers and the null stream handle; every call below is refused before anything is
    launched)."""
    import torch
    x = torch.zeros((1, 5, 8, 12, 4), dtype=torch.bfloat16)
    with pytest.raises(v.VaeError) as e:          # 5 frames fold causally by 2 -> 3, not 2
        v.vae_space_to_depth(x, 2, 2, 2, torch.zeros((1, 2, 4, 6, 32), dtype=torch.bfloat16),
                             stream=0)
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    with pytest.raises(v.VaeError) as e:          # 12 columns do not fold by 5
        v.vae_space_to_depth(x, 1, 2, 5, torch.zeros((1, 5, 4, 2, 40), dtype=torch.bfloat16),
                             stream=0)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED and e.value.info["axis"] == 3
    assert e.value.info["required_multiple"] == 5
    with pytest.raises(v.VaeError) as e:          # factors below 1
        v.vae_space_to_depth(x, 0, 2, 2, torch.zeros((1, 3, 4, 6, 32), dtype=torch.bfloat16),
                             stream=0)
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    with pytest.raises(v.VaeError) as e:          # y aliasing x
        v.vae_space_to_depth(x, 1, 1, 1, x, stream=0)
    assert e.value.status == v.VAE_ERR_INVALID_ARG


def test_groupnorm_noalloc_refuses_beyond_its_scratch(v):
    """vae_groupnorm_silu_noalloc holds 8 MiB of scratch per GPU: a call that needs more is
    refused on the host, before any device work, with the byte counts in the error info. The
    tensor descriptors are never dereferenced."""
    # 16 samples of [16, 256, 256, 256]: 1024 statistics blocks x 16 x 32 groups x 24 bytes; two
    # far-apart stand-in addresses, so that the tensors do not overlap
    big = v.vae_tensor_t(1 << 40, v.VAE_DTYPE_BF16, 0, 16, 16, 256, 256, 256)
    y = v.vae_tensor_t(1 << 41, v.VAE_DTYPE_BF16, 0, 16, 16, 256, 256, 256)
    st = v.LIB.vae_groupnorm_silu_noalloc(ctypes.byref(big), None, 1, 32, 1e-6, None, None, 1,
                                          ctypes.byref(y), None)
    assert st == v.VAE_ERR_UNSUPPORTED
    info = v.last_error_info()
    assert info["min_width"] == 8 << 20 and info["extent"] > 8 << 20
    assert b"noalloc" in v.LIB.vae_last_error()


def test_strided_conv_plan_rules(v):
    """A plan's strided downsampler (VAE_OP_CONV_DOWN): strides of 1 or 2 with sh == sw, padding
    after the image only with stride 2, and input extents of whole strides."""
    def plan(**kw):
        op = {"op": "conv_down", "cin": 32, "cout": 64, "st": 2, "sh": 2, "sw": 2, "pad": "around"}
        op.update(kw)
        return [op, {"op": "gn_silu"}, {"op": "conv", "cin": 64, "cout": 32, "f32_out": True}]
    ptrs = [_FakePtr(i) for i in range(6)]
    dec = v.Decoder(v.VAE_DTYPE_BF16, 32, 32, 1e-6, plan(), ptrs)
    assert dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 5, 8, 8, 32),
                                            (1, 1, 1))) > 0
    with pytest.raises(v.VaeError) as e:          # 7 rows are not whole strides of 2
        dec.workspace_size(v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 5, 7, 8, 32), (1, 1, 1)))
    assert e.value.status == v.VAE_ERR_INVALID_ARG and e.value.info["axis"] == 2
    dec.close()
    for bad, status in [(dict(sh=3, sw=3), v.VAE_ERR_UNSUPPORTED),
                        (dict(sh=2, sw=1), v.VAE_ERR_UNSUPPORTED),
                        (dict(st=1, sh=1, sw=1, pad="after"), v.VAE_ERR_UNSUPPORTED),
                        (dict(cin=16), v.VAE_ERR_INVALID_ARG)]:
        with pytest.raises(v.VaeError) as e:
            v.Decoder(v.VAE_DTYPE_BF16, 32, 32, 1e-6, plan(**bad), ptrs)
        assert e.value.status == status, bad


def test_decode_status_argument_checks(v):
    """vae_decode_status checks its arguments on the host before touching the device."""
    import vae_synth
    spec = vae_synth.LTX2_TINY
    n_ptr = sum({"conv": 2, "res": 8, "gn_silu": 2}.get(op["op"], 0) for op in spec["layers"])
    dec = v.Decoder(v.VAE_DTYPE_BF16, 128, 32, 1e-6, spec["layers"],
                    [_FakePtr(i) for i in range(n_ptr)])
    desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, (1, 2, 4, 6, 128), spec["scale"])
    need = dec.workspace_size(desc)
    flags = ctypes.c_int32()
    assert v.LIB.vae_decode_status(dec._h, ctypes.byref(desc), None, need, ctypes.byref(flags),
                                   None) == v.VAE_ERR_INVALID_ARG
    assert v.LIB.vae_decode_status(dec._h, ctypes.byref(desc), ctypes.c_void_p(1 << 40),
                                   need - 1, ctypes.byref(flags), None) == v.VAE_ERR_WORKSPACE
    assert v.LIB.vae_decode_status(dec._h, ctypes.byref(desc), ctypes.c_void_p(1 << 40), need,
                                   None, None) == v.VAE_ERR_INVALID_ARG
    dec.close()


def _plan_decoder(v, spec, flags=0):
    n_ptr = sum({"conv": 2, "res": 8, "res_rms": 8, "gn_silu": 2, "rms_silu": 2, "attn": 6}
                .get(op["op"], 0) for op in spec["layers"])
    lc = v.latent_channels(spec)
    layers = [dict(op) for op in spec["layers"]]
    first = next(op for op in layers if op["op"] == "conv")
    first["cin"] = lc
    return v.Decoder(v.VAE_DTYPE_BF16, lc, spec["groups"], spec["eps"], layers,
                     [_FakePtr(i) for i in range(n_ptr)], flags=flags)


def test_clip_frames_rules_and_workspace(v):
    """A clip-by-clip decode takes plans whose every op is local in time (convs, RMS norms, frame
    attention, upsamplings); a GroupNorm plan is refused. Its workspace holds one clip's
    activations plus headroom and the carried frames: at the Wan 720p plan (21 latent frames) a
    clip of 2 needs far less than the whole decode, and a clip at least as long as the latent
    decodes at once, with the whole decode's workspace."""
    import vae_synth
    spec = vae_synth.WAN_720P
    dec = _plan_decoder(v, spec, flags=v.VAE_DECODE_F16_OPERANDS)
    shape = (1, 21, 44, 80, v.latent_channels(spec))
    desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, shape, spec["scale"], patches=(1, 4))
    whole = dec.workspace_size(desc)
    dec.set_clip_frames(2)
    clip2 = dec.workspace_size(desc)
    assert clip2 < whole / 4
    # each of the three buffers holds at least a later clip's 8 frames of the 256-channel
    # activation at 352 x 640 (2 bytes a value at least)
    assert clip2 >= 3 * 8 * 352 * 640 * 256 * 2
    dec.set_clip_frames(21)
    assert dec.workspace_size(desc) == whole
    dec.set_clip_frames(0)
    assert dec.workspace_size(desc) == whole
    # the overlap-blend mode ignores the setting
    ob = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, shape, spec["scale"], tile=(32, 32),
                       stride=(28, 28))
    b = dec.workspace_size(ob)
    dec.set_clip_frames(2)
    assert dec.workspace_size(ob) == b
    with pytest.raises(v.VaeError) as e:
        dec.set_clip_frames(-1)
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    dec.close()
    for name in ("ltx2_tiny", "mixed_rms_gn"):
        g = _plan_decoder(v, vae_synth.WORKLOADS[name])
        with pytest.raises(v.VaeError) as e:       # GroupNorm statistics span every frame
            g.set_clip_frames(1)
        assert e.value.status == v.VAE_ERR_UNSUPPORTED
        g.set_clip_frames(0)
        g.close()
