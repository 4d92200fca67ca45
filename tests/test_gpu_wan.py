"""GPU parity of the Wan-shaped path (RMS norm, frame attention, the whole decode) against the CPU
oracle, through the C ABI.

Tolerances:
- RMS norm: fp32 output relative max-abs <= 1e-4; bf16 / fp16 outputs half an ulp of the reference
  plus 1e-4 relative;
- frame attention: the operands are bf16 (normalised input, projections) and fp16 (q, k, v,
  softmax weights), about 2^-9 relative each. The attention's own contribution y - x is held to
  relative max-abs <= 2e-2, and y to PSNR >= 50 dB;
- decodes: PSNR >= 50 dB and max-abs <= 2e-2 against the fp64 oracle.
"""
import functools

import numpy as np
import pytest

import oracle
import vae_synth
from _util import (ndhwc, dev, host, rel_max_abs, psnr, bf16_round_bound, f16_round_bound,
                   round_f16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def v():
    import torch
    import video_diffusion_vae_amd as v
    assert torch.cuda.is_available()
    return v


RMS_CASES = [
    # (N, T, H, W, C), in dtype, out dtype, silu
    ((1, 3, 5, 7, 128), "f32", "bf16", True),
    ((2, 2, 4, 6, 1024), "f32", "f16", True),
    ((1, 2, 3, 5, 256), "bf16", "f32", False),
    ((1, 1, 7, 9, 32), "f32", "f32", True),
    ((1, 2, 4, 4, 2048), "f32", "bf16", False),
    ((1, 3, 3, 3, 512), "bf16", "bf16", True),
    # fp16 inputs: the first conv of a residual block stores its output in fp16
    ((1, 3, 5, 7, 128), "f16", "bf16", True),
    ((1, 2, 3, 5, 1024), "f16", "f16", True),
]


@pytest.mark.parametrize("case", RMS_CASES)
def test_rmsnorm_matches_oracle(v, case):
    import torch
    shape, idt, odt, act = case
    n, t, h, w, c = shape
    x = ndhwc(vae_synth.normal((n, c, t, h, w), [50, c], scale=1.7, mean=0.2, dtype=idt))
    if idt == "f16":
        x = round_f16(x)             # the oracle sees exactly the values the GPU reads
    gamma = vae_synth.normal((c,), [51, c], scale=0.2, mean=1.0)
    beta = vae_synth.normal((c,), [52, c], scale=0.1)
    ref = oracle.rms_norm(x, 1e-6, gamma, beta)
    if act:
        ref = oracle.silu(ref)
    xd = dev(x, idt)
    y = torch.empty(xd.shape, device="cuda", dtype={"bf16": torch.bfloat16, "f16": torch.float16,
                                                    "f32": torch.float32}[odt])
    v.vae_rmsnorm_silu(xd, 1e-6, torch.as_tensor(gamma, device="cuda"),
                       torch.as_tensor(beta, device="cuda"), act, y)
    torch.cuda.synchronize()
    got = host(y)
    if odt == "f32":
        assert rel_max_abs(got, ref) <= 1e-4
    else:
        bound = bf16_round_bound(ref) if odt == "bf16" else f16_round_bound(ref)
        assert np.all(np.abs(got - ref) <= bound + 1e-4 * np.abs(ref).max())


def _attn_params(c, seed):
    g = vae_synth.normal((c,), [53, seed, 0], scale=0.2, mean=1.0)
    b = vae_synth.normal((c,), [53, seed, 1], scale=0.1)
    wq = vae_synth.normal((3 * c, c), [53, seed, 2], scale=1 / np.sqrt(c), dtype="bf16")
    bq = vae_synth.normal((3 * c,), [53, seed, 3], scale=0.1)
    wo = vae_synth.normal((c, c), [53, seed, 4], scale=1 / np.sqrt(c), dtype="bf16")
    bo = vae_synth.normal((c,), [53, seed, 5], scale=0.1)
    return g, b, wq, bq, wo, bo


ATTN_CASES = [
    # (N, T, H, W, C): frames of 15, 128, 143 and 300 positions (ragged GEMM tiles and K tails)
    (1, 2, 3, 5, 64),
    (1, 3, 8, 16, 32),
    (2, 1, 11, 13, 128),
    (1, 2, 15, 20, 256),
]


@pytest.mark.parametrize("shape", ATTN_CASES)
def test_frame_attention_matches_oracle(v, shape):
    import torch
    n, t, h, w, c = shape
    x = ndhwc(vae_synth.normal((n, c, t, h, w), [54, c, h]))
    g, b, wq, bq, wo, bo = _attn_params(c, h)
    ref = oracle.frame_attention(x, 1e-6, g, b, wq, bq, wo, bo)
    T = lambda a, dt=torch.float32: torch.as_tensor(np.asarray(a, np.float32)).to("cuda", dt)
    xd = dev(x, "f32")
    y = torch.full_like(xd, float("nan"))
    v.vae_frame_attention(xd, 1e-6, T(g), T(b), T(wq, torch.bfloat16), T(bq),
                          T(wo, torch.bfloat16), T(bo), y)
    torch.cuda.synchronize()
    got = host(y)
    assert np.all(np.isfinite(got))
    assert rel_max_abs(got - x, ref - x) <= 2e-2
    assert psnr(got, ref) >= 50.0
    # in place (y = x) gives the same result bit for bit
    v.vae_frame_attention(xd, 1e-6, T(g), T(b), T(wq, torch.bfloat16), T(bq),
                          T(wo, torch.bfloat16), T(bo), xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, y)


@functools.lru_cache(maxsize=None)
def _params(name):
    return vae_synth.decoder_params(vae_synth.WORKLOADS[name], affine_seed=5)


@functools.lru_cache(maxsize=None)
def _oracle(name, mode, tt=(0, 0)):
    spec = vae_synth.WORKLOADS[name]
    z = ndhwc(vae_synth.latent(spec))
    if mode == "patch":
        return oracle.decode(spec, z, _params(name))
    return oracle.decode_overlap_blend(spec, z, _params(name), spec["overlap_tile"],
                                       spec["overlap_stride"], spec["scale"], tt[0], tt[1])


def _decode(v, name, mode, patches=(1, 1), operands="f16", repeat=1, tt=(0, 0), clip=0,
            launch=None):
    import torch
    spec = vae_synth.WORKLOADS[name]
    z = v.pad_latent(ndhwc(vae_synth.latent(spec)), spec)
    dec = v.upload_decoder(spec, _params(name), operands=operands)
    if clip:
        dec.set_clip_frames(clip)
    if launch is not None:
        dec.set_launch(launch)
    zd = dev(z, "bf16")
    if mode == "patch":
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, z.shape, spec["scale"], patches=patches)
    else:
        desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, z.shape, spec["scale"],
                             tile=spec["overlap_tile"], stride=spec["overlap_stride"],
                             tile_t=tt[0], stride_t=tt[1])
    ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(repeat):
        out = torch.full(oracle.output_shape(spec, ndhwc(vae_synth.latent(spec)).shape),
                         float("nan"), device="cuda", dtype=torch.float32)
        dec.vae_decode_tiled(zd, desc, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    dec.close()
    return outs if repeat > 1 else outs[0]


@pytest.mark.parametrize("operands", ["f16", "split"])
@pytest.mark.parametrize("name,mode,patches", [("wan_tiny", "patch", (2, 2)),
                                               ("wan_tiny", "overlap", (1, 1)),
                                               ("wan_small", "patch", (1, 2)),
                                               ("wan_small", "patch", (1, 1)),
                                               ("wan_small", "overlap", (1, 1)),
                                               # an RMS residual block feeding a GroupNorm
                                               ("mixed_rms_gn", "patch", (1, 2)),
                                               ("mixed_rms_gn", "patch", (1, 1)),
                                               ("mixed_rms_gn", "overlap", (1, 1))])
def test_wan_shaped_decode(v, name, mode, patches, operands):
    got = host(_decode(v, name, mode, patches, operands))
    ref = _oracle(name, mode)
    assert got.shape == ref.shape
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


def test_wan_shaped_decode_temporal_tiles(v):
    """Overlap-blend tiles in T as well as in space: the 3 latent frames of wan_tiny as clips
    [0,2) [1,3) [2,3) (output frames [0,5) [4,9) [8,9)), each decoded alone with its own causal
    start, per-frame attention and RMS norms, then blended."""
    got = host(_decode(v, "wan_tiny", "overlap", tt=(2, 1)))
    ref = _oracle("wan_tiny", "overlap", (2, 1))
    assert got.shape == ref.shape == (1, 9, 64, 96, 3)
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


@pytest.mark.parametrize("name,clip,patches,per_patch", [("wan_tiny", 1, (1, 1), False),
                                                          ("wan_tiny", 2, (2, 2), False),
                                                          ("wan_tiny", 2, (2, 2), True),
                                                          ("wan_tiny", 1, (2, 2), True),
                                                          ("wan_small", 1, (1, 2), False)])
def test_wan_shaped_decode_clip_by_clip(v, name, clip, patches, per_patch):
    """The patch-halo decode in causal clips of `clip` latent frames, every causal conv carrying
    its last two input frames into the next clip: the whole decode of the oracle, at the bf16
    bar (wan_tiny's 3 frames as [0,1) [1,2) [2,3) or [0,2) [2,3); wan_small's 2 as one-frame
    clips)."""
    got = host(_decode(v, name, "patch", patches, clip=clip,
                       launch=v.VAE_LAUNCH_PER_PATCH if per_patch else None))
    ref = _oracle(name, "patch")
    assert got.shape == ref.shape
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


def test_wan_shaped_decode_is_deterministic(v):
    import torch
    a, b = _decode(v, "wan_tiny", "patch", (2, 2), repeat=2)
    assert torch.equal(a, b)


def test_wan_720p_one_frame_every_value(v):
    """The full-width Wan-shaped 720p plan on one latent frame ([1,48,1,44,80] ->
    [1,1,704,1280,3]) in 1 x 4 width patches: the attention gathers all 3520 positions of the
    frame, and every output value is compared with the oracle's whole decode (the overlap mode
    is covered at the small sizes above; its oracle at this size takes over a minute)."""
    got = host(_decode(v, "wan_720p_1f", "patch", (1, 4)))
    ref = _oracle("wan_720p_1f", "patch")
    assert got.shape == (1, 1, 704, 1280, 3)
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)


@pytest.mark.parametrize("clip", [0, 2])
def test_wan_720p_six_frames_against_golden(v, clip):
    """The full-width Wan-shaped 720p plan on six latent frames ([1,48,6,44,80] ->
    [1,21,704,1280,3]) in 1 x 4 width patches, at the pixels the oracle's fp64 decode stored
    (tests/golden/make_wan_720p_samples.py): both temporal upsamplings and the causal temporal taps
    at full spatial size. With clip = 2 the same decode runs as three causal clips of two latent
    frames (output frames [0,5) [5,13) [13,21)), the frames carried at full size."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "wan_720p_6f_whole_samples.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    g = np.load(path)
    out = _decode(v, "wan_720p_6f", "patch", (1, 4), clip=clip)
    assert tuple(out.shape) == tuple(int(d) for d in g["shape"])
    pos = g["positions"]
    got = out[0, pos[:, 0], pos[:, 1], pos[:, 2], :].double().cpu().numpy()
    ref = g["values"]
    assert np.all(np.isfinite(got))
    p = 10 * np.log10((float(g["out_max"]) - float(g["out_min"])) ** 2 / np.mean((got - ref) ** 2))
    m = float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)
    o = out.double()
    assert abs(float(o.mean()) - float(g["out_mean"])) <= 1e-3 * float(g["out_std"])
    assert abs(float(o.std()) / float(g["out_std"]) - 1.0) <= 1e-3


def test_wan_720p_first_frames_of_the_full_decode_every_value(v):
    """The full 21-frame Wan-shaped 720p decode ([1,48,21,44,80] -> [1,81,704,1280,3]) in 1 x 4
    width patches. Its output frames 0..4 depend only on latent frames 0 and 1: the convs are
    causal, the norms per position, the attention per frame and the temporal upsamplers causal
    (pinned on the CPU by test_oracle_decoder's first-frames test). So the oracle decodes those two
    latent frames alone (about half a minute on the CPU), and every one of the 13.5M values of
    frames 0..4 of the full GPU decode is held to the bf16 bar: frames past frame 0 of a full-T
    decode, at every value."""
    spec = vae_synth.WAN_720P
    got = _decode(v, "wan_720p", "patch", (1, 4))
    assert tuple(got.shape) == (1, 81, 704, 1280, 3)
    got = got[:, :5].double().cpu().numpy()
    z = ndhwc(vae_synth.latent(spec))[:, :2]
    ref = oracle.decode(vae_synth.with_latent(spec, (1, 48, 2, 44, 80), "wan_720p_2f"), z,
                        _params("wan_720p"))
    assert ref.shape == got.shape
    p, m = psnr(got, ref), float(np.abs(got - ref).max())
    assert p >= 50.0 and m <= 2e-2, (p, m)
