"""GPU parity of each C-ABI call against the CPU oracle, on seeded inputs.

Tolerances:
- fp32 paths: relative max-abs <= 1e-4;
- bf16 inputs with fp32 output: products are exact in fp32, so the same 1e-4;
- bf16 outputs: half a bf16 ulp of the reference plus 1e-4 relative (one rounding per store);
  fp16 outputs: half an fp16 ulp plus 1e-4 relative;
- fp16 inputs: the operands are exact (fp16 x, bf16 weights scaled by 2^10 into fp16), so fp32
  outputs are held to 1e-4 relative;
- integer/permutation work (upsampling): bit-exact.
"""
import numpy as np
import pytest

import oracle
import vae_synth
from _util import ndhwc, dev, host, rel_max_abs, bf16_round_bound, f16_round_bound, round_f16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def v():
    import torch
    import video_diffusion_vae_amd as v
    assert torch.cuda.is_available()
    return v


def _conv_inputs(shape, cin, cout, dtype, seed):
    n, t, h, w = shape
    x = ndhwc(vae_synth.normal((n, cin, t, h, w), [10, seed], dtype=dtype))
    wt = vae_synth.normal((cout, cin, 3, 3, 3), [11, seed], scale=1 / np.sqrt(27 * cin), dtype=dtype)
    b = vae_synth.normal((cout,), [12, seed], scale=0.1)
    r = ndhwc(vae_synth.normal((n, cout, t, h, w), [13, seed], dtype=dtype))
    return x, np.asarray(wt, np.float64), np.asarray(b, np.float64), r


CONV_CASES = [
    # (N, T, H, W), Cin, Cout, in dtype, out dtype, residual, box (t0,t1,h0,h1,w0,w1) or None
    ((1, 3, 9, 17), 32, 64, "bf16", "bf16", False, None),
    ((1, 5, 10, 20), 64, 128, "bf16", "f32", True, None),
    ((2, 2, 8, 16), 32, 48, "bf16", "f32", False, None),
    ((1, 4, 11, 23), 128, 256, "bf16", "bf16", True, (1, 4, 2, 9, 5, 15)),
    ((1, 1, 7, 5), 96, 128, "bf16", "bf16", False, None),
    ((1, 6, 16, 32), 256, 384, "bf16", "f32", True, (0, 6, 0, 16, 8, 24)),
    ((1, 3, 9, 19), 64, 256, "f32", "f32", True, None),
    ((2, 4, 6, 17), 32, 64, "f32", "bf16", False, (0, 3, 1, 6, 3, 17)),
    ((1, 2, 8, 16), 128, 52, "f32", "f32", False, None),
]


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv3d_mfma_matches_oracle(v, case):
    """bf16 weights on the matrix cores. An fp32 input is the operand after its nearest-even
    rounding to bf16, so the reference convolves that rounded input."""
    import torch
    (n, t, h, w), cin, cout, idt, odt, use_res, bx = case
    x, wt, b, r = _conv_inputs((n, t, h, w), cin, cout, "bf16", CONV_CASES.index(case))
    if idt == "f32":   # an fp32 activation with finer values than bf16
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [14, cin], scale=1e-3))
        ref = oracle.causal_conv3d(vae_synth.round_bf16(x), wt, b)
    else:
        ref = oracle.causal_conv3d(x, wt, b)
    if use_res:
        ref = ref + r
    xd = dev(x, idt)
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    rd = dev(r, odt) if use_res else None
    y = torch.full((n, t, h, w, cout), 7.0, device="cuda",
                   dtype=torch.float32 if odt == "f32" else torch.bfloat16)
    v.vae_conv3d_causal(xd, wd, bd, rd, y, bx)
    torch.cuda.synchronize()
    got = host(y)
    if bx is None:
        bx = (0, t, 0, h, 0, w)
    sl = (slice(None), slice(bx[0], bx[1]), slice(bx[2], bx[3]), slice(bx[4], bx[5]))
    mask = np.zeros(got.shape, bool)
    mask[sl] = True
    assert np.all(got[~mask] == 7.0), "conv wrote outside its box"
    g, rf = got[sl], ref[sl]
    if odt == "f32":
        assert rel_max_abs(g, rf) <= 1e-4
    else:
        assert np.all(np.abs(g - rf) <= bf16_round_bound(rf) + 1e-4 * np.abs(rf).max())


# Boxes 10, 12 or 20 positions wide, deep in T (one width quarter of the first decoder stages):
# the extents make the launch pick a narrow block shape, which stages through one tile buffer
# and stores through the LDS epilogue. (N, T, H, W), Cin, Cout, in, out, residual, box; the
# comment names the block shape the extents select.
NARROW_CASES = [
    ((1, 16, 22, 10), 64, 128, "bf16", "f32", True, None),              # 16 x 8 x 2
    ((1, 16, 12, 12), 64, 128, "bf16", "bf16", False, None),            # 16 x 4 x 4
    ((1, 4, 16, 12), 64, 128, "bf16", "f32", True, None),               # 4 x 16 x 4
    ((2, 16, 9, 10), 32, 64, "bf16", "bf16", True, None),               # 16 x 8 x 2, N = 2
    ((1, 17, 13, 30), 64, 128, "bf16", "f32", True, (1, 17, 2, 13, 10, 20)),   # 16 x 8 x 2 box
    ((1, 16, 12, 12), 64, 48, "f32", "f32", False, None),               # 16 x 4 x 4, Cout 48
    # 32-wide channel tiles: staging rounds of 8 units, then a last round of 4 or 3
    ((1, 16, 22, 10), 96, 32, "bf16", "f32", True, None),               # 16 x 8 x 2, Cout 32
    ((1, 4, 16, 12), 64, 12, "bf16", "bf16", False, None),              # 4 x 16 x 4, Cout 12
]


@pytest.mark.parametrize("case", NARROW_CASES)
def test_conv3d_narrow_blocks(v, case):
    """The narrow block shapes against the oracle, with standard and packed weights (which must
    agree bit for bit); nothing outside the box is written."""
    import torch
    (n, t, h, w), cin, cout, idt, odt, use_res, bx = case
    x, wt, b, r = _conv_inputs((n, t, h, w), cin, cout, "bf16", 40 + NARROW_CASES.index(case))
    if idt == "f32":
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [15, cin], scale=1e-3))
        ref = oracle.causal_conv3d(vae_synth.round_bf16(x), wt, b)
    else:
        ref = oracle.causal_conv3d(x, wt, b)
    if use_res:
        ref = ref + r
    xd = dev(x, idt)
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    rd = dev(r, odt) if use_res else None
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    y = torch.full((n, t, h, w, cout), 7.0, device="cuda", dtype=tdt)
    v.vae_conv3d_causal(xd, wd, bd, rd, y, bx)
    yp = torch.full_like(y, 7.0)
    v.vae_conv3d_causal(xd, v.vae_conv_weight_pack(wd).view(torch.bfloat16), bd, rd, yp, bx,
                        v.VAE_CONV_PACKED_WEIGHTS)
    torch.cuda.synchronize()
    assert torch.equal(y, yp)
    got = host(y)
    bx = bx or (0, t, 0, h, 0, w)
    sl = (slice(None), slice(bx[0], bx[1]), slice(bx[2], bx[3]), slice(bx[4], bx[5]))
    mask = np.zeros(got.shape, bool)
    mask[sl] = True
    assert np.all(got[~mask] == 7.0), "conv wrote outside its box"
    g, rf = got[sl], ref[sl]
    if odt == "f32":
        assert rel_max_abs(g, rf) <= 1e-4
    else:
        assert np.all(np.abs(g - rf) <= bf16_round_bound(rf) + 1e-4 * np.abs(rf).max())


# Split over K (VAE_CONV_SPLIT_K): launches too small to fill the chip. (N, T, H, W), Cin,
# C (after the depth-to-space), d2s factors, in, out, GroupNorm groups (0: none), residual
SPLIT_K_CASES = [
    ((1, 16, 22, 10), 256, 256, (1, 1, 1), "bf16", "f32", 32, True),    # S0-quarter-like, 4 splits
    ((1, 16, 22, 10), 128, 64, (2, 2, 2), "f16", "f16", 0, False),      # up-conv-like, d2s
    ((1, 4, 6, 10), 128, 32, (2, 2, 2), "bf16", "f32", 8, False),       # d2s + statistics
    ((1, 3, 9, 17), 256, 48, (1, 1, 1), "f32", "f32", 0, True),         # fp32 in, Cout 48
    ((2, 16, 9, 10), 128, 128, (1, 1, 1), "bf16", "bf16", 32, False),   # N = 2, 2 splits
]


@pytest.mark.parametrize("case", SPLIT_K_CASES)
def test_conv3d_split_k(v, case):
    """A conv split over its input-channel chunks (one launch of partial sums, one that adds them
    in split order and runs the epilogue): matches the oracle like the unsplit conv, differs
    from it only by fp32 summation order, gathers the same statistics, and is deterministic."""
    import torch
    (n, t, h, w), cin, c, (st, sh, sw), idt, odt, groups, use_res = case
    cout = c * st * sh * sw
    x, wt, b, _ = _conv_inputs((n, t, h, w), cin, cout, "bf16", 70 + SPLIT_K_CASES.index(case))
    if idt == "f32":
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [18, cin], scale=1e-3))
        xin = vae_synth.round_bf16(x).astype(np.float64)
    elif idt == "f16":
        x = round_f16(x + ndhwc(vae_synth.normal((n, cin, t, h, w), [18, cin], scale=1e-3)))
        xin = x
    else:
        xin = x
    yshape = (n, st * t - (st - 1), sh * h, sw * w, c)
    r = ndhwc(vae_synth.normal((yshape[0], c) + yshape[1:4], [19, cin], dtype="bf16")) \
        if use_res else None
    ref = oracle.depth_to_space(oracle.causal_conv3d(xin, wt, b), st, sh, sw)
    if use_res:
        ref = ref + r
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[odt]
    xd = dev(x, idt)
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    flags = 0
    if idt == "f16":
        wd = v.vae_conv_weight_pack_f16(wd).view(torch.bfloat16)
        flags = v.VAE_CONV_PACKED_F16_WEIGHTS
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    rd = dev(r, odt) if use_res else None
    outs, stats = [], []
    for fl in (flags | v.VAE_CONV_SPLIT_K, flags | v.VAE_CONV_SPLIT_K, flags):
        y = torch.full(yshape, 7.0, device="cuda", dtype=tdt)
        mr = torch.zeros((n, max(groups, 1), 2), dtype=torch.float32, device="cuda")
        v.vae_conv3d_causal_fused(xd, wd, bd, rd, y, None, fl, d2s=(st, sh, sw),
                                  gn_groups=groups, gn_eps=1e-6, gn_mean_rstd=mr)
        outs.append(y)
        stats.append(mr)
    torch.cuda.synchronize()
    # the split needs scratch beyond the statistics: the query grows with the flag
    assert v.vae_conv3d_causal_fused_workspace(xd, wd, outs[0], None, (st, sh, sw), groups,
                                               flags=flags) < \
        v.vae_conv3d_causal_fused_workspace(xd, wd, outs[0], None, (st, sh, sw), groups,
                                            flags=flags | v.VAE_CONV_SPLIT_K)
    assert torch.equal(outs[0], outs[1]), "split conv is not deterministic"
    got, unsplit = host(outs[0]), host(outs[2])
    if odt == "f32":
        assert rel_max_abs(got, ref) <= 1e-4
        assert rel_max_abs(got, unsplit) <= 1e-5
    else:
        bound = bf16_round_bound(ref) if odt == "bf16" else f16_round_bound(ref)
        assert np.all(np.abs(got - ref) <= bound + 1e-4 * np.abs(ref).max())
        assert np.all(np.abs(got - unsplit) <= 2 * bound + 1e-5 * np.abs(ref).max())
    if groups:
        cnt, mean, m2 = oracle.group_moments(got, groups)      # of y as stored
        gm = stats[0].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(gm[..., 0], mean, rtol=0, atol=1e-5 * np.sqrt(m2 / cnt).max())
        np.testing.assert_allclose(gm[..., 1], 1 / np.sqrt(m2 / cnt + 1e-6), rtol=1e-5)


# Strided causal convs: (N, T, H, W), Cin, Cout, strides, pad, in dtype, out dtype, weights
# ("packed": the matrix-core kernel, "std": the direct kernel), residual dtype (None: none), box
STRIDED_CASES = [
    ((1, 5, 16, 24), 64, 128, (2, 2, 2), "around", "bf16", "f32", "packed", "f32", None),
    ((1, 4, 18, 14), 32, 64, (1, 2, 2), "after", "bf16", "bf16", "packed", None, None),
    ((2, 3, 9, 11), 64, 32, (2, 1, 1), "around", "f16", "f16", "packed", None, None),
    ((1, 7, 20, 20), 128, 256, (2, 2, 2), "around", "bf16", "f32", "packed", None,
     (1, 4, 2, 10, 0, 6)),
    ((1, 6, 16, 16), 64, 128, (2, 2, 2), "after", "bf16", "bf16", "packed", "f32", None),
    ((1, 4, 12, 12), 32, 48, (1, 1, 1), "around", "bf16", "f32", "packed", None, None),
    ((1, 3, 8, 10), 48, 20, (2, 2, 2), "after", "f32", "f32", "std", None, None),
    ((1, 4, 7, 9), 16, 24, (2, 2, 2), "around", "bf16", "bf16", "std", "bf16", None),
]


@pytest.mark.parametrize("case", STRIDED_CASES)
def test_conv3d_strided_matches_oracle(v, case):
    """vae_conv3d_causal_strided against oracle.strided_causal_conv3d (an fp32 x is compared
    after its rounding to the bf16 operand on the matrix cores, unrounded on the direct path);
    nothing outside the box is written, and the result is deterministic."""
    import torch
    (n, t, h, w), cin, cout, stride, pad, idt, odt, wk, rdt, bx = case
    seed = 50 + STRIDED_CASES.index(case)
    x, wt, b, _ = _conv_inputs((n, t, h, w), cin, cout, "bf16", seed)
    if idt == "f32":
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [15, cin], scale=1e-3))
    elif idt == "f16":
        x = round_f16(x + ndhwc(vae_synth.normal((n, cin, t, h, w), [15, cin], scale=1e-3)))
    pads = {"around": ((1, 1), (1, 1)), "after": ((0, 1), (0, 1))}[pad]
    ref = oracle.strided_causal_conv3d(x, wt, b, stride, pads)
    yshape = ref.shape
    r = None
    if rdt:
        r = ndhwc(vae_synth.normal((yshape[0], cout) + yshape[1:4], [16, seed], dtype="bf16"))
        ref = ref + r
    xd = dev(x, idt)
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    flags = 0
    if wk == "packed":
        if idt == "f16":
            wd, flags = v.vae_conv_weight_pack_f16(wd), v.VAE_CONV_PACKED_F16_WEIGHTS
        else:
            wd, flags = v.vae_conv_weight_pack(wd), v.VAE_CONV_PACKED_WEIGHTS
        wd = wd.view(torch.bfloat16)
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    rd = dev(r, rdt) if rdt else None
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[odt]
    ys = []
    for _ in range(2):
        y = torch.full(yshape, 7.0, device="cuda", dtype=tdt)
        v.vae_conv3d_causal_strided(xd, wd, bd, rd, y, stride, pad, bx, flags)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    got = host(ys[0])
    bx = bx or (0, yshape[1], 0, yshape[2], 0, yshape[3])
    sl = (slice(None), slice(bx[0], bx[1]), slice(bx[2], bx[3]), slice(bx[4], bx[5]))
    mask = np.zeros(got.shape, bool)
    mask[sl] = True
    assert np.all(got[~mask] == 7.0), "wrote outside the box"
    g, rf = got[sl], ref[sl]
    if odt == "f32":
        assert rel_max_abs(g, rf) <= 1e-4
    else:
        bound = bf16_round_bound(rf) if odt == "bf16" else f16_round_bound(rf)
        assert np.all(np.abs(g - rf) <= bound + 1e-4 * np.abs(rf).max())


def test_conv3d_strided_argument_rules(v):
    import torch
    x = torch.zeros((1, 5, 8, 8, 32), device="cuda", dtype=torch.bfloat16)
    w = torch.zeros((64, 3, 3, 3, 32), device="cuda", dtype=torch.bfloat16)
    y = torch.zeros((1, 3, 4, 4, 64), device="cuda", dtype=torch.bfloat16)
    v.vae_conv3d_causal_strided(x, w, None, None, y, (2, 2, 2), "around")
    with pytest.raises(v.VaeError) as e:           # wrong output extent
        v.vae_conv3d_causal_strided(x, w, None, None, y[:, :2].contiguous(), (2, 2, 2), "around")
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    with pytest.raises(v.VaeError) as e:           # packed weights off the matrix-core rules
        v.vae_conv3d_causal_strided(x.float(), w, None, None, y.float(), (2, 2, 2), "around",
                                    flags=v.VAE_CONV_PACKED_WEIGHTS)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    with pytest.raises(v.VaeError) as e:           # stride 0
        v.vae_conv3d_causal_strided(x, w, None, None, y, (0, 2, 2), "around")
    assert e.value.status == v.VAE_ERR_INVALID_ARG


CONV_GN_CASES = [
    # (N, T, H, W), Cin, Cout, groups, in dtype, out dtype, residual, box
    ((1, 3, 9, 17), 32, 128, 32, "bf16", "f32", False, None),            # 4 channels per group
    ((2, 4, 6, 20), 64, 256, 32, "bf16", "bf16", True, None),            # 8, two samples
    ((1, 5, 10, 20), 32, 512, 32, "bf16", "f32", True, (1, 5, 2, 9, 3, 17)),  # 16, in a box
    ((1, 2, 5, 9), 64, 1024, 32, "bf16", "f32", False, None),            # 32
    ((1, 3, 9, 19), 64, 64, 8, "f32", "f32", False, None),               # 64-wide tiles
    ((1, 3, 6, 9), 32, 64, 32, "bf16", "f32", False, None),              # 2: separate pass
    ((1, 3, 6, 9), 16, 32, 8, "bf16", "f32", True, None),                # direct conv path
    # Cout 32 in a 64-wide tile: one wave's channels all past Cout
    ((1, 3, 8, 20), 64, 32, 8, "bf16", "f32", True, None),
    ((1, 3, 8, 16), 32, 32, 4, "bf16", "bf16", False, (0, 3, 1, 8, 2, 15)),  # in a box
]


@pytest.mark.parametrize("case", CONV_GN_CASES)
def test_conv3d_gn_statistics(v, case):
    """Conv plus the GroupNorm statistics of its stored output over the box. The epilogue gathers
    them on the MFMA path (4-32 channels per group). Other shapes take a separate pass.
    Checks:
     - y is bit-identical to vae_conv3d_causal's;
     - mean/rstd match the oracle's two-pass statistics of the oracle conv;
     - mean/rstd match the separate statistics pass run over the same y."""
    import torch
    (n, t, h, w), cin, cout, groups, idt, odt, use_res, bx = case
    x, wt, b, r = _conv_inputs((n, t, h, w), cin, cout, "bf16", 60 + CONV_GN_CASES.index(case))
    if idt == "f32":
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [16, cin], scale=1e-3))
        ref = oracle.causal_conv3d(vae_synth.round_bf16(x), wt, b)
    else:
        ref = oracle.causal_conv3d(x, wt, b)
    if use_res:
        ref = ref + r
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    xd = dev(x, idt)
    wd = v.conv_weight_layout(wt, torch.bfloat16 if cin % 32 == 0 else torch.float32, "cuda")
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    rd = dev(r, odt) if use_res else None
    y = torch.full((n, t, h, w, cout), 7.0, device="cuda", dtype=tdt)
    mr = torch.zeros((n, groups, 2), dtype=torch.float32, device="cuda")
    v.vae_conv3d_causal_fused(xd, wd, bd, rd, y, bx, gn_groups=groups, gn_eps=1e-6,
                              gn_mean_rstd=mr)
    y0 = torch.full_like(y, 7.0)
    v.vae_conv3d_causal(xd, wd, bd, rd, y0, bx)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    bx = bx or (0, t, 0, h, 0, w)
    sl = (slice(None), slice(bx[0], bx[1]), slice(bx[2], bx[3]), slice(bx[4], bx[5]))
    rf = ref[sl] if odt == "f32" else vae_synth.round_bf16(ref[sl]).astype(np.float64)
    cnt, mean, m2 = oracle.group_moments(rf, groups)
    var = m2 / cnt
    got = mr.cpu().numpy().astype(np.float64)
    tol = 1e-4 if odt == "f32" else 1e-3
    assert np.all(np.abs(got[..., 0] - mean) <= tol * np.sqrt(var) + 1e-6)
    np.testing.assert_allclose(got[..., 1], 1 / np.sqrt(var + 1e-6), rtol=tol)
    # the separate statistics pass over the same y
    part = torch.zeros((1, n, groups, 3), dtype=torch.float64, device="cuda")
    v.vae_groupnorm_stats(y, [bx], groups, part)
    mr2 = torch.zeros_like(mr)
    v.vae_groupnorm_combine(part, 1, n, groups, 1e-6, mr2)
    torch.cuda.synchronize()
    np.testing.assert_allclose(got, mr2.cpu().numpy(), rtol=2e-5, atol=1e-6)


CONV_D2S_CASES = [
    # (N, T, H, W), Cin, C (channels after d2s), (st, sh, sw), in dtype, out dtype, split,
    # box, GroupNorm groups (0: none)
    ((1, 3, 5, 9), 64, 32, (2, 2, 2), "bf16", "f32", False, None, 8),
    ((1, 4, 6, 7), 32, 64, (2, 2, 2), "f32", "f32", True, (1, 4, 1, 6, 2, 7), 16),
    ((2, 2, 4, 10), 64, 32, (1, 2, 2), "bf16", "bf16", False, None, 4),
    ((1, 1, 3, 5), 32, 128, (2, 2, 2), "bf16", "f32", False, None, 32),
    ((1, 3, 4, 6), 32, 3, (1, 4, 4), "f32", "f32", True, None, 0),      # unpatchify-like
    ((1, 2, 3, 5), 32, 3, (1, 4, 1), "bf16", "f32", False, None, 0),    # channel-wise stores
]


@pytest.mark.parametrize("case", CONV_D2S_CASES)
def test_conv3d_fused_depth_to_space(v, case):
    """Conv whose epilogue writes the depth-to-space of its output (with the causal frame drop),
    optionally with the GroupNorm statistics of that result.
    Checks:
     - it matches the oracle conv followed by the oracle depth-to-space;
     - it is bit-identical to the GPU conv followed by vae_upsample;
     - the statistics match the oracle's over the part of y written."""
    import torch
    (n, t, h, w), cin, c, (st, sh, sw), idt, odt, split, bx, groups = case
    cout = c * st * sh * sw
    x, wt, b, _ = _conv_inputs((n, t, h, w), cin, cout, "bf16", 80 + CONV_D2S_CASES.index(case))
    if idt == "f32":
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [17, cin], scale=1e-3))
    if split:
        hi = vae_synth.round_bf16(x).astype(np.float64)
        xin = hi + vae_synth.round_bf16(x - hi).astype(np.float64)
    else:
        xin = vae_synth.round_bf16(x).astype(np.float64)
    full = oracle.causal_conv3d(xin, wt, b)
    bx_ = bx or (0, t, 0, h, 0, w)
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    xd = dev(x, idt)
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    flags = v.VAE_CONV_SPLIT_FP32 if split else 0
    yshape = (n, st * t - (st - 1), sh * h, sw * w, c)
    y = torch.full(yshape, 7.0, device="cuda", dtype=tdt)
    mr = torch.zeros((n, max(groups, 1), 2), dtype=torch.float32, device="cuda")
    v.vae_conv3d_causal_fused(xd, wd, bd, None, y, bx, flags, d2s=(st, sh, sw),
                              gn_groups=groups, gn_eps=1e-6, gn_mean_rstd=mr)
    # the two-step GPU path: conv into a full tensor, then depth-to-space of the box
    y1 = torch.full((n, t, h, w, cout), 0.0, device="cuda", dtype=tdt)
    v.vae_conv3d_causal(xd, wd, bd, None, y1, bx, flags)
    y2 = torch.full(yshape, 7.0, device="cuda", dtype=tdt)
    v.vae_upsample(y1, bx, v.VAE_UPSAMPLE_D2S, st, sh, sw, y2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    # against the oracle, over the part of y this call writes
    ref = oracle.depth_to_space(full, st, sh, sw)
    t0 = max(0, st * bx_[0] - (st - 1))
    sl = (slice(None), slice(t0, st * bx_[1] - (st - 1)), slice(sh * bx_[2], sh * bx_[3]),
          slice(sw * bx_[4], sw * bx_[5]))
    got = host(y)
    mask = np.zeros(got.shape, bool)
    mask[sl] = True
    assert np.all(got[~mask] == 7.0), "wrote outside the box's image"
    g, rf = got[sl], ref[sl]
    if odt == "f32":
        assert rel_max_abs(g, rf) <= 1e-4
    else:
        assert np.all(np.abs(g - rf) <= bf16_round_bound(rf) + 1e-4 * np.abs(rf).max())
    if groups:
        rs = rf if odt == "f32" else vae_synth.round_bf16(rf).astype(np.float64)
        cnt, mean, m2 = oracle.group_moments(rs, groups)
        var = m2 / cnt
        gm = mr.cpu().numpy().astype(np.float64)
        tol = 1e-4 if odt == "f32" else 1e-3
        assert np.all(np.abs(gm[..., 0] - mean) <= tol * np.sqrt(var) + 1e-6)
        np.testing.assert_allclose(gm[..., 1], 1 / np.sqrt(var + 1e-6), rtol=tol)


@pytest.mark.parametrize("shape,cin,cout,box", [((1, 3, 9, 19), 64, 256, None),
                                                 ((1, 5, 7, 33), 32, 48, (1, 5, 0, 7, 4, 30))])
def test_conv3d_split_operands(v, shape, cin, cout, box):
    """VAE_CONV_SPLIT_FP32: an fp32 input applied as bf16 hi + lo. The reference convolves
    hi + lo, which carries about 16 significant bits of x, so fp32 output matches it at 1e-4."""
    import torch
    n, t, h, w = shape
    x, wt, b, _ = _conv_inputs(shape, cin, cout, "bf16", 40 + cin)
    x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [15, cin], scale=3e-3))
    hi = vae_synth.round_bf16(x).astype(np.float64)
    lo = vae_synth.round_bf16(x - hi).astype(np.float64)
    ref = oracle.causal_conv3d(hi + lo, wt, b)
    y = torch.full((n, t, h, w, cout), 7.0, device="cuda", dtype=torch.float32)
    v.vae_conv3d_causal(dev(x, "f32"), v.conv_weight_layout(wt, torch.bfloat16, "cuda"),
                        torch.as_tensor(b, dtype=torch.float32, device="cuda"), None, y, box,
                        flags=v.VAE_CONV_SPLIT_FP32)
    torch.cuda.synchronize()
    got = host(y)
    bx = box or (0, t, 0, h, 0, w)
    sl = (slice(None), slice(bx[0], bx[1]), slice(bx[2], bx[3]), slice(bx[4], bx[5]))
    assert rel_max_abs(got[sl], ref[sl]) <= 1e-4
    # the single-rounding result is measurably further from the exact fp32 convolution
    exact = oracle.causal_conv3d(x, wt, b)[sl]
    y1 = torch.empty_like(y)
    v.vae_conv3d_causal(dev(x, "f32"), v.conv_weight_layout(wt, torch.bfloat16, "cuda"),
                        torch.as_tensor(b, dtype=torch.float32, device="cuda"), None, y1, box)
    torch.cuda.synchronize()
    assert rel_max_abs(got[sl], exact) < 0.25 * rel_max_abs(host(y1)[sl], exact)


@pytest.mark.parametrize("dtype,cin", [("f32", 16), ("f32", 32), ("bf16", 16), ("bf16", 24)])
def test_conv3d_direct_paths(v, dtype, cin):
    import torch
    x, wt, b, _ = _conv_inputs((1, 3, 6, 9), cin, 20, dtype, cin)
    ref = oracle.causal_conv3d(x, wt, b)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.empty((1, 3, 6, 9, 20), device="cuda", dtype=torch.float32)
    v.vae_conv3d_causal(dev(x, dtype), v.conv_weight_layout(wt, tdt, "cuda"),
                        torch.as_tensor(b, dtype=torch.float32, device="cuda"), None, y)
    torch.cuda.synchronize()
    assert rel_max_abs(host(y), ref) <= 1e-4


def test_conv3d_rejects_bad_arguments(v):
    import torch
    x = torch.zeros((1, 2, 4, 4, 32), device="cuda", dtype=torch.bfloat16)
    w = torch.zeros((16, 3, 3, 3, 32), device="cuda", dtype=torch.bfloat16)
    y = torch.zeros((1, 2, 4, 5, 16), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(v.VaeError) as e:
        v.vae_conv3d_causal(x, w, None, None, y)
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    y = torch.zeros((1, 2, 4, 4, 16), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(v.VaeError):
        v.vae_conv3d_causal(x, w, None, None, y, (0, 3, 0, 4, 0, 4))


GN_CASES = [
    # in dtype > out dtype, (N, T, H, W, C), groups, patch cuts (h cuts, w cuts)
    ("f32>f32", (1, 5, 32, 32, 32), 8, ([], [16])),
    ("f32>f32", (2, 3, 16, 16, 64), 32, ([7], [3, 11])),
    ("bf16>bf16", (1, 3, 12, 20, 128), 32, ([5], [10])),
    ("bf16>bf16", (1, 2, 8, 10, 1024), 32, ([], [1, 5, 9])),
    ("bf16>bf16", (1, 4, 9, 13, 256), 32, ([], [])),
    ("f32>f32", (1, 3, 8, 8, 32), 32, ([4], [4])),
    ("f32>bf16", (1, 3, 11, 20, 128), 32, ([], [5, 10, 15])),
    ("f32>bf16", (1, 2, 8, 10, 1024), 32, ([4], [])),
    ("bf16>f32", (1, 2, 6, 7, 256), 32, ([3], [])),
    ("f32>f16", (1, 3, 11, 20, 128), 32, ([], [5, 10, 15])),
    ("bf16>f16", (1, 2, 8, 10, 256), 32, ([4], [])),
    # fp16 inputs: the first conv of a residual block stores its output in fp16
    ("f16>bf16", (1, 3, 12, 20, 128), 32, ([5], [10])),
    ("f16>f16", (1, 2, 8, 10, 1024), 32, ([], [1, 5, 9])),
    ("f16>f32", (1, 2, 6, 7, 256), 32, ([3], [])),
]


def _boxes(shape, cuts):
    _, t, h, w, _ = shape
    hs = [0] + cuts[0] + [h]
    ws = [0] + cuts[1] + [w]
    return [(0, t, hs[i], hs[i + 1], ws[j], ws[j + 1])
            for i in range(len(hs) - 1) for j in range(len(ws) - 1)]


@pytest.mark.parametrize("case", GN_CASES)
def test_groupnorm_silu_patch_stats(v, case):
    import torch
    dts, shape, groups, cuts = case
    idt, odt = dts.split(">")
    n, t, h, w, c = shape
    x = ndhwc(vae_synth.normal((n, c, t, h, w), [20, c, h], scale=1.5, mean=0.3, dtype=idt))
    if idt == "f16":
        x = round_f16(x)             # the oracle sees exactly the values the GPU reads
    gamma = vae_synth.normal((c,), [21, c], scale=0.2, mean=1.0)
    beta = vae_synth.normal((c,), [22, c], scale=0.1)
    ref = oracle.silu(oracle.group_norm(x, groups, 1e-6, gamma, beta))
    boxes = _boxes(shape, cuts)
    xd = dev(x, idt)
    y = torch.empty(xd.shape, device="cuda",
                    dtype={"bf16": torch.bfloat16, "f16": torch.float16}.get(odt, torch.float32))
    g_d, b_d = torch.as_tensor(gamma, device="cuda"), torch.as_tensor(beta, device="cuda")
    v.vae_groupnorm_silu(xd, boxes, groups, 1e-6, g_d, b_d, True, y)
    torch.cuda.synchronize()
    got = host(y)
    if odt == "f32":
        assert rel_max_abs(got, ref) <= 1e-4
    else:
        bound = bf16_round_bound(ref) if odt == "bf16" else f16_round_bound(ref)
        assert np.all(np.abs(got - ref) <= bound + 1e-4 * np.abs(ref).max())
    # determinism: the same call gives a bitwise identical result (in place when dtypes match)
    y2 = xd if idt == odt else torch.empty_like(y)
    v.vae_groupnorm_silu(xd, boxes, groups, 1e-6, g_d, b_d, True, y2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y)


def test_groupnorm_stats_export_and_combine(v):
    import torch
    shape, groups = (2, 3, 10, 12, 64), 32
    x = ndhwc(vae_synth.normal((2, 64, 3, 10, 12), [23], scale=2.0, mean=-1.0))
    boxes = _boxes(shape, ([4], [5, 9]))
    xd = dev(x, "f32")
    part = torch.zeros((len(boxes), 2, groups, 3), dtype=torch.float64, device="cuda")
    v.vae_groupnorm_stats(xd, boxes, groups, part)
    mr = torch.zeros((2, groups, 2), dtype=torch.float32, device="cuda")
    v.vae_groupnorm_combine(part, len(boxes), 2, groups, 1e-6, mr)
    torch.cuda.synchronize()
    p = part.cpu().numpy()
    for i, bx in enumerate(boxes):
        cnt, mean, m2 = oracle.group_moments(x[:, bx[0]:bx[1], bx[2]:bx[3], bx[4]:bx[5]], groups)
        assert np.array_equal(p[i, :, :, 0], cnt.astype(np.float64))
        np.testing.assert_allclose(p[i, :, :, 1], mean, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(p[i, :, :, 2], m2, rtol=1e-5)
    cnt, mean, m2 = oracle.group_moments(x, groups)
    got = mr.cpu().numpy()
    np.testing.assert_allclose(got[..., 0], mean, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(got[..., 1], 1 / np.sqrt(m2 / cnt + 1e-6), rtol=1e-5)
    # apply with the exported statistics equals the one-call path
    y1 = torch.empty_like(xd)
    v.vae_groupnorm_apply(xd, None, groups, mr, None, None, False, y1)
    ref = oracle.group_norm(x, groups, 1e-6)
    torch.cuda.synchronize()
    assert rel_max_abs(host(y1), ref) <= 1e-4


def test_groupnorm_large_mean_stress(v):
    """fp32 input with mean 1e3 and std 1: the case random weights never produce."""
    import torch
    x = ndhwc(vae_synth.normal((1, 32, 4, 16, 24), [24], scale=1.0, mean=1e3))
    ref = oracle.group_norm(x, 8, 1e-6)
    xd = dev(x, "f32")
    y = torch.empty_like(xd)
    v.vae_groupnorm_silu(xd, _boxes((1, 4, 16, 24, 32), ([], [12])), 8, 1e-6, None, None, False, y)
    torch.cuda.synchronize()
    assert rel_max_abs(host(y), ref) <= 1e-4


UP_CASES = [
    ("bf16", (1, 3, 4, 5, 64), "d2s", (2, 2, 2), None),
    ("bf16", (2, 2, 3, 4, 32), "d2s", (2, 2, 2), (1, 2, 0, 3, 1, 4)),
    ("f32", (1, 3, 4, 6, 48), "d2s", (1, 4, 4), None),
    ("f32", (1, 2, 5, 3, 12), "d2s", (2, 1, 1), None),
    ("bf16", (1, 2, 3, 4, 16), "nearest", (1, 2, 2), None),
    ("f32", (1, 1, 3, 3, 4), "nearest", (1, 2, 3), (0, 1, 1, 3, 0, 2)),
    ("f16", (1, 3, 4, 5, 64), "d2s", (2, 2, 2), None),
    ("f16", (1, 2, 3, 4, 16), "nearest", (1, 2, 2), (0, 2, 1, 3, 0, 4)),
    # depth-to-space whose output rows come in runs of at least 128 bytes (sw * C): the kernel
    # that goes by input rows, with ragged 512-vector slices and boxes
    ("f32", (1, 3, 4, 6, 256), "d2s", (2, 2, 2), None),
    ("bf16", (1, 2, 3, 5, 512), "d2s", (2, 2, 2), None),
    ("bf16", (2, 3, 4, 6, 256), "d2s", (1, 2, 2), (1, 3, 1, 4, 2, 6)),
    ("f16", (1, 2, 3, 4, 512), "d2s", (2, 2, 2), (0, 2, 0, 3, 1, 3)),
    ("f32", (1, 2, 3, 70, 128), "d2s", (1, 1, 2), None),
]


@pytest.mark.parametrize("case", UP_CASES)
def test_upsample_bit_exact(v, case):
    import torch
    dtype, shape, mode, (st, sh, sw), bx = case
    n, t, h, w, c = shape
    x = ndhwc(vae_synth.normal((n, c, t, h, w), [25, c], dtype=dtype))
    if dtype == "f16":
        x = round_f16(x)
    if mode == "d2s":
        ref = oracle.depth_to_space(x, st, sh, sw)
        m = v.VAE_UPSAMPLE_D2S
    else:
        ref = oracle.nearest_upsample(x, sh, sw)
        m = v.VAE_UPSAMPLE_NEAREST
    xd = dev(x, dtype)
    y = torch.full(ref.shape, -3.0, device="cuda", dtype=xd.dtype)
    v.vae_upsample(xd, bx, m, st, sh, sw, y)
    torch.cuda.synchronize()
    got = host(y)
    if bx is None:
        assert np.array_equal(got, ref)
    else:
        t0, t1, h0, h1, w0, w1 = bx
        lo_t = max(0, st * t0 - (st - 1))
        sl = (slice(None), slice(lo_t, st * t1 - (st - 1)), slice(sh * h0, sh * h1),
              slice(sw * w0, sw * w1))
        assert np.array_equal(got[sl], ref[sl])
        mask = np.zeros(got.shape, bool)
        mask[sl] = True
        assert np.all(got[~mask] == -3.0)


@pytest.mark.parametrize("grid", [((16, 16), (14, 14), (22, 40), (2, 4, 4), 2, (0, 0)),
                                  ((4, 5), (3, 2), (9, 11), (1, 3, 2), 2, (0, 0)),
                                  ((8, 8), (8, 8), (8, 8), (1, 2, 2), 2, (0, 0)),
                                  # temporal tiles: clips [0,3) [2,5) [4,5); 3 shared frames
                                  ((4, 5), (3, 2), (9, 11), (2, 3, 2), 5, (3, 2)),
                                  ((0, 0), (0, 0), (5, 7), (4, 1, 1), 7, (4, 1))])
def test_tile_merge_matches_oracle(v, grid):
    import torch
    tile, stride, (lh, lw), scale, lt, (tt, stt) = grid
    desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, (1, lt, lh, lw, 3), scale, tile=tile,
                         stride=stride, tile_t=tt, stride_t=stt)
    tiles = v.vae_tile_split(desc)
    ref_tiles = oracle.overlap_tiles(lt, lh, lw, tile, stride, scale, tt, stt)
    assert len(tiles) == len(ref_tiles)
    out_shape = (1, 1 + (lt - 1) * scale[0], lh * scale[1], lw * scale[2], 3)
    outs = []
    for k, tl in enumerate(ref_tiles):
        o = tl["out"]
        outs.append(vae_synth.normal((1, o[1] - o[0], o[3] - o[2], o[5] - o[4], 3), [26, k])
                    .astype(np.float64))
    ref = oracle.merge_tiles(outs, ref_tiles, out_shape)
    out = torch.full(out_shape, 5.0, device="cuda", dtype=torch.float32)
    for k, tl in enumerate(tiles):
        flags = (v.VAE_MERGE_ZERO if k == 0 else 0) | \
                (v.VAE_MERGE_FINALIZE if k == len(tiles) - 1 else 0)
        v.vae_tile_merge(dev(outs[k], "f32"), tl, desc, out, flags)
    torch.cuda.synchronize()
    assert rel_max_abs(host(out), ref) <= 1e-5


PACKED_CASES = [
    # (N, T, H, W), Cin, Cout, input dtype, split fp32 operands
    ((1, 3, 9, 19), 64, 256, "bf16", False),
    ((2, 2, 8, 16), 32, 48, "f32", False),
    ((1, 2, 8, 16), 128, 52, "f32", False),
    ((1, 5, 10, 12), 96, 128, "bf16", False),
    # 2x8x16 blocks: the packed path stages through the ring of frame slots
    ((1, 4, 16, 32), 96, 128, "bf16", False),          # three chunks
    ((1, 5, 16, 32), 64, 256, "bf16", False),          # a ragged last frame block, two Cout tiles
    ((1, 4, 16, 32), 64, 128, "f32", True),            # split: four 16-channel chunks
    ((2, 3, 8, 16), 32, 48, "f32", True),              # 64-wide tiles, two samples
    # 4x8x8 and 4x4x16 blocks: six-frame tiles in a ring of eight slots
    ((1, 7, 8, 24), 96, 128, "bf16", False),           # 4x8x8, ragged last frame block
    ((1, 8, 12, 32), 64, 256, "bf16", False),          # 4x4x16, ragged rows
    ((1, 6, 16, 8), 32, 128, "f32", True),             # 4x8x8, split
    # Cout a multiple of 32 but not of the tile: waves whose 32 channels are all past Cout
    ((1, 3, 8, 16), 64, 32, "bf16", False),            # 64-wide tile, one wave past Cout
    ((1, 4, 8, 24), 32, 96, "bf16", False),            # second 64-wide tile half used
    ((1, 3, 9, 16), 64, 160, "bf16", False),           # 128-wide tiles, three waves past Cout
    ((1, 3, 8, 16), 32, 96, "f32", True),              # split, 64-wide tiles
]


@pytest.mark.parametrize("case", PACKED_CASES)
def test_conv3d_packed_weights_bitwise_equal(v, case):
    """Packed weights only change the load layout (and, for 2x8x16 blocks, the staging order):
    the result must be bitwise identical to the standard layout, and match the oracle."""
    import torch
    (n, t, h, w), cin, cout, idt, split = case
    x, wt, b, _ = _conv_inputs((n, t, h, w), cin, cout, "bf16", 60 + PACKED_CASES.index(case))
    if idt == "f32":
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [18, cin], scale=1e-3))
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    packed = v.vae_conv_weight_pack(wd)
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    y0 = torch.empty((n, t, h, w, cout), device="cuda", dtype=torch.float32)
    y1 = torch.empty_like(y0)
    xd = dev(x, idt)
    sf = v.VAE_CONV_SPLIT_FP32 if split else 0
    v.vae_conv3d_causal(xd, wd, bd, None, y0, flags=sf)
    v.vae_conv3d_causal(xd, packed.view(torch.bfloat16), bd, None, y1,
                        flags=v.VAE_CONV_PACKED_WEIGHTS | sf)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    if split:
        hi = vae_synth.round_bf16(x).astype(np.float64)
        xin = hi + vae_synth.round_bf16(x - hi).astype(np.float64)
    else:
        xin = vae_synth.round_bf16(x).astype(np.float64)
    assert rel_max_abs(host(y1), oracle.causal_conv3d(xin, wt, b)) <= 1e-4


F16_IN_CASES = [
    # (N, T, H, W), Cin, Cout, out dtype, residual, box
    ((1, 3, 9, 17), 32, 64, "f32", False, None),
    ((1, 5, 10, 20), 64, 128, "f32", True, None),
    ((2, 2, 8, 16), 32, 48, "f32", False, None),                    # staged epilogue
    ((1, 4, 11, 23), 128, 256, "bf16", True, (1, 4, 2, 9, 5, 15)),
    ((1, 2, 8, 16), 128, 52, "f32", True, None),
    ((1, 1, 7, 5), 96, 128, "f32", False, None),
]


@pytest.mark.parametrize("case", F16_IN_CASES)
def test_conv3d_f16_input(v, case):
    """An fp16 input runs v_mfma_f32_32x32x16_f16 against the bf16 weights converted to fp16
    (scaled by 2^10, then the sums by 2^-10): the operands are exact, so the result is the
    oracle's conv of the fp16 values up to fp32 summation. Standard-layout and fp16-packed
    weights give bitwise equal results."""
    import torch
    (n, t, h, w), cin, cout, odt, use_res, bx = case
    x, wt, b, r = _conv_inputs((n, t, h, w), cin, cout, "bf16", 80 + F16_IN_CASES.index(case))
    # an fp32 activation with finer values than bf16, rounded once to fp16
    x = round_f16(x + ndhwc(vae_synth.normal((n, cin, t, h, w), [15, cin], scale=1e-3)))
    ref = oracle.causal_conv3d(x, wt, b)
    if use_res:
        ref = ref + r
    xd = dev(x, "f16")
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    rd = dev(r, odt) if use_res else None
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    y = torch.full((n, t, h, w, cout), 7.0, device="cuda", dtype=tdt)
    v.vae_conv3d_causal(xd, wd, bd, rd, y, bx)
    yp = torch.full_like(y, 7.0)
    wp = v.vae_conv_weight_pack_f16(wd).view(torch.bfloat16)
    v.vae_conv3d_causal(xd, wp, bd, rd, yp, bx, flags=v.VAE_CONV_PACKED_F16_WEIGHTS)
    torch.cuda.synchronize()
    assert torch.equal(y, yp)
    got = host(y)
    bx = bx or (0, t, 0, h, 0, w)
    sl = (slice(None), slice(bx[0], bx[1]), slice(bx[2], bx[3]), slice(bx[4], bx[5]))
    mask = np.zeros(got.shape, bool)
    mask[sl] = True
    assert np.all(got[~mask] == 7.0), "conv wrote outside its box"
    g, rf = got[sl], ref[sl]
    if odt == "f32":
        assert rel_max_abs(g, rf) <= 1e-4
    else:
        assert np.all(np.abs(g - rf) <= bf16_round_bound(rf) + 1e-4 * np.abs(rf).max())


F16_OUT_CASES = [
    # (N, T, H, W), Cin, Cout, residual dtype (None = no residual), input dtype
    ((1, 3, 9, 17), 64, 128, "f32", "bf16"),   # direct epilogue, fp32 residual stream
    ((1, 4, 8, 16), 32, 64, "f16", "bf16"),
    ((2, 2, 8, 16), 32, 48, "f32", "bf16"),    # staged epilogue
    ((1, 2, 5, 9), 128, 256, None, "bf16"),
    ((1, 3, 8, 16), 64, 128, None, "f16"),     # fp16 in, fp16 out (a conv feeding a conv)
]


@pytest.mark.parametrize("case", F16_OUT_CASES)
def test_conv3d_f16_output_handoff(v, case):
    """A conv that stores fp16 (the operand hand-off to an fp16-input conv), with an fp32 or fp16
    residual: one nearest-even rounding of the fp32 sum."""
    import torch
    (n, t, h, w), cin, cout, rdt, idt = case
    x, wt, b, r = _conv_inputs((n, t, h, w), cin, cout, "bf16", 90 + F16_OUT_CASES.index(case))
    if idt == "f16":
        x = round_f16(x + ndhwc(vae_synth.normal((n, cin, t, h, w), [17, cin], scale=1e-3)))
    if rdt == "f16":
        r = round_f16(r)
    ref = oracle.causal_conv3d(x, wt, b) + (r if rdt else 0.0)
    y = torch.full((n, t, h, w, cout), 7.0, device="cuda", dtype=torch.float16)
    v.vae_conv3d_causal(dev(x, idt), v.conv_weight_layout(wt, torch.bfloat16, "cuda"),
                        torch.as_tensor(b, dtype=torch.float32, device="cuda"),
                        dev(r, rdt) if rdt else None, y)
    torch.cuda.synchronize()
    got = host(y)
    assert np.all(np.abs(got - ref) <= f16_round_bound(ref) + 1e-4 * np.abs(ref).max())


def test_conv3d_f16_argument_rules(v):
    import torch
    x16 = torch.zeros((1, 2, 4, 4, 32), device="cuda", dtype=torch.float16)
    xb = torch.zeros((1, 2, 4, 4, 32), device="cuda", dtype=torch.bfloat16)
    w = torch.zeros((32, 3, 3, 3, 32), device="cuda", dtype=torch.bfloat16)
    y = torch.zeros((1, 2, 4, 4, 32), device="cuda", dtype=torch.float32)
    y16 = torch.zeros((1, 2, 4, 4, 32), device="cuda", dtype=torch.float16)
    with pytest.raises(v.VaeError) as e:        # bf16-packed weights with an fp16 input
        v.vae_conv3d_causal(x16, v.vae_conv_weight_pack(w).view(torch.bfloat16), None, None, y,
                            flags=v.VAE_CONV_PACKED_WEIGHTS)
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    with pytest.raises(v.VaeError) as e:        # fp16-packed weights with a bf16 input
        v.vae_conv3d_causal(xb, v.vae_conv_weight_pack_f16(w).view(torch.bfloat16), None, None, y,
                            flags=v.VAE_CONV_PACKED_F16_WEIGHTS)
    assert e.value.status == v.VAE_ERR_INVALID_ARG
    x32 = torch.zeros((1, 2, 4, 4, 32), device="cuda", dtype=torch.float32)
    with pytest.raises(v.VaeError) as e:        # an fp16 output needs a 2-byte input
        v.vae_conv3d_causal(x32, w, None, None, y16)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED
    x20 = torch.zeros((1, 2, 4, 4, 20), device="cuda", dtype=torch.float16)
    with pytest.raises(v.VaeError) as e:        # fp16 needs the MFMA path (Cin % 32)
        v.vae_conv3d_causal(x20, w[..., :20].contiguous(), None, None, y)
    assert e.value.status == v.VAE_ERR_UNSUPPORTED



IN_UP_CASES = [
    # (N, T, h, w) of x before the upsampling, Cin, Cout, dtype, (sh, sw), box in the upsampled grid
    ((1, 3, 5, 9), 64, 128, "bf16", (2, 2), None),
    ((1, 2, 4, 6), 32, 64, "f16", (2, 2), (0, 2, 1, 7, 3, 12)),
    ((2, 2, 3, 8), 64, 96, "f32", (2, 1), None),
    ((1, 3, 4, 4), 32, 48, "bf16", (4, 4), None),
    ((1, 4, 6, 10), 64, 32, "f16", (2, 2), (1, 4, 0, 12, 0, 20)),
]


@pytest.mark.parametrize("case", IN_UP_CASES)
def test_conv3d_folded_nearest_upsampling(v, case):
    """A conv reading the nearest upsampling of x while it stages its input equals
    vae_upsample(NEAREST) followed by the conv, bit for bit (same operands, same order)."""
    import torch
    (n, t, h, w), cin, cout, dt, (sh, sw), bx = case
    x, wt, b, _ = _conv_inputs((n, t, h, w), cin, cout, "bf16", 95 + IN_UP_CASES.index(case))
    if dt == "f16":
        x = round_f16(x + ndhwc(vae_synth.normal((n, cin, t, h, w), [18, cin], scale=1e-3)))
    elif dt == "f32":
        x = x + ndhwc(vae_synth.normal((n, cin, t, h, w), [18, cin], scale=1e-3))
    xd = dev(x, dt)
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    xu = torch.empty((n, t, h * sh, w * sw, cin), device="cuda", dtype=xd.dtype)
    v.vae_upsample(xd, None, v.VAE_UPSAMPLE_NEAREST, 1, sh, sw, xu)
    y0 = torch.full((n, t, h * sh, w * sw, cout), 7.0, device="cuda", dtype=torch.float32)
    y1 = torch.full_like(y0, 7.0)
    v.vae_conv3d_causal(xu, wd, bd, None, y0, bx)
    v.vae_conv3d_causal_fused(xd, wd, bd, None, y1, bx, in_up=(sh, sw))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    # and both are the oracle's conv of the upsampled input
    xin = vae_synth.round_bf16(x).astype(np.float64) if dt == "f32" else x
    ref = oracle.causal_conv3d(oracle.nearest_upsample(xin, sh, sw), wt, b)
    bx = bx or (0, t, 0, h * sh, 0, w * sw)
    sl = (slice(None), slice(bx[0], bx[1]), slice(bx[2], bx[3]), slice(bx[4], bx[5]))
    assert rel_max_abs(host(y1)[sl], ref[sl]) <= 1e-4


# GroupNorm + SiLU applied by the conv while it stages its input (in_scale_shift).
# (N, T, H, W), Cin, C (after the depth-to-space), d2s, x dtype, operand dtype, y dtype,
# residual, box, groups, split over K
NORM_IN_CASES = [
    ((1, 3, 9, 17), 64, 128, (1, 1, 1), "f32", "bf16", "f32", True, None, 32, False),
    ((1, 5, 10, 20), 128, 128, (1, 1, 1), "f16", "bf16", "f16", False, None, 32, False),
    ((2, 2, 8, 16), 32, 48, (1, 1, 1), "f32", "f16", "f32", False, None, 8, False),   # conv_out
    ((1, 4, 11, 23), 256, 256, (1, 1, 1), "f16", "bf16", "f32", True, (1, 4, 2, 9, 5, 15), 32,
     False),
    ((1, 3, 6, 10), 128, 32, (2, 2, 2), "f32", "bf16", "f32", False, None, 32, False),  # d2s
    ((1, 16, 22, 10), 256, 256, (1, 1, 1), "f16", "bf16", "f32", True, None, 32, True),
    ((1, 2, 16, 4), 64, 64, (1, 1, 1), "f32", "bf16", "bf16", False, None, 16, False),  # narrow
]


@pytest.mark.parametrize("case", NORM_IN_CASES)
def test_conv3d_applies_input_groupnorm(v, case):
    """The conv reads silu(x * scale + shift) (the scale and shift of a GroupNorm from
    vae_groupnorm_scale_shift), rounding it to its operand type while staging: bit for bit what
    vae_groupnorm_apply into a bf16 (fp16) tensor followed by the conv gives, and the oracle's
    conv of the rounded normalised input. The oracle normalises in fp64, the kernel in fp32, so
    at a rounding tie the two operands can land one bf16 (fp16) step apart: about one operand in
    2^15, each moving an output by about |w| * ulp(z) (2e-5 of the largest output here). The
    oracle bar is therefore 3e-4 relative for fp32 outputs (some ten such steps on one output);
    the bit-exact match with the separate pass pins the kernel's own rounding."""
    import torch
    (n, t, h, w), cin, c, (st, sh, sw), xdt, odt, ydt, use_res, bx, groups, splitk = case
    k = NORM_IN_CASES.index(case)
    cout = c * st * sh * sw
    _, wt, b, _ = _conv_inputs((n, t, h, w), cin, cout, "bf16", 120 + k)
    x = ndhwc(vae_synth.normal((n, cin, t, h, w), [121, k], scale=1.7, mean=0.4))
    if xdt == "f16":
        x = round_f16(x)
    gamma = vae_synth.normal((cin,), [122, k], scale=0.3, mean=1.0)
    beta = vae_synth.normal((cin,), [123, k], scale=0.2)
    cnt, mean, m2 = oracle.group_moments(x, groups)
    var = m2 / cnt
    eps = 1e-6
    z = oracle.silu(oracle.normalize_with(x, groups, mean, var, eps, gamma, beta))
    zop = vae_synth.round_bf16(z).astype(np.float64) if odt == "bf16" else round_f16(z)
    yshape = (n, st * t - (st - 1), sh * h, sw * w, c)
    r = ndhwc(vae_synth.normal((n, c) + yshape[1:4], [124, k], dtype="bf16")) if use_res else None
    ref = oracle.depth_to_space(oracle.causal_conv3d(zop, wt, b), st, sh, sw)
    if use_res:
        ref = ref + r
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    xd = dev(x, xdt)
    wd = v.conv_weight_layout(wt, torch.bfloat16, "cuda")
    if odt == "f16":
        wp = v.vae_conv_weight_pack_f16(wd).view(torch.bfloat16)
        flags = v.VAE_CONV_PACKED_F16_WEIGHTS
    else:
        wp = v.vae_conv_weight_pack(wd).view(torch.bfloat16)
        flags = v.VAE_CONV_PACKED_WEIGHTS
    if splitk:
        flags |= v.VAE_CONV_SPLIT_K
    bd = torch.as_tensor(b, dtype=torch.float32, device="cuda")
    rd = dev(r, ydt) if use_res else None
    mr = torch.as_tensor(np.stack([mean, 1 / np.sqrt(var + eps)], -1), dtype=torch.float32,
                         device="cuda")
    gd = torch.as_tensor(gamma, dtype=torch.float32, device="cuda")
    bt = torch.as_tensor(beta, dtype=torch.float32, device="cuda")
    ab = torch.empty((n, cin, 2), dtype=torch.float32, device="cuda")
    v.vae_groupnorm_scale_shift(mr, cin, groups, gd, bt, ab)
    # the separate pass: the normalised tensor in the operand dtype, then the conv
    g = torch.empty(xd.shape, dtype=tdt[odt], device="cuda")
    v.vae_groupnorm_apply(xd, None, groups, mr, gd, bt, True, g)
    outs = []
    for src, fused in ((g, False), (xd, True)):
        y = torch.full(yshape, 7.0, device="cuda", dtype=tdt[ydt])
        v.vae_conv3d_causal_fused(src, wp, bd, rd, y, bx, flags, d2s=(st, sh, sw),
                                  in_scale_shift=ab if fused else None)
        outs.append(y)
    torch.cuda.synchronize()
    sep, got = host(outs[0]), host(outs[1])
    diff = np.abs(sep - got)
    assert torch.equal(outs[0], outs[1]), \
        f"fused input norm differs from the separate pass: {int((diff > 0).sum())} values, " \
        f"max {diff.max():.3g}; vs oracle {rel_max_abs(got, ref):.3g} (fused), " \
        f"{rel_max_abs(sep, ref):.3g} (separate)"
    if bx is None:
        g_, rf = got, ref
    else:   # the box in the conv's input grid; y's frames and columns scale with the factors
        t0, t1 = max(0, st * bx[0] - (st - 1)), st * bx[1] - (st - 1)
        sl = (slice(None), slice(t0, t1), slice(sh * bx[2], sh * bx[3]),
              slice(sw * bx[4], sw * bx[5]))
        mask = np.zeros(got.shape, bool)
        mask[sl] = True
        assert np.all(got[~mask] == 7.0), "conv wrote outside its box"
        g_, rf = got[sl], ref[sl]
    if ydt == "f32":
        assert rel_max_abs(g_, rf) <= 3e-4
    else:
        bound = bf16_round_bound(rf) if ydt == "bf16" else f16_round_bound(rf)
        assert np.all(np.abs(g_ - rf) <= bound + 3e-4 * np.abs(rf).max())


def test_groupnorm_scale_shift_matches_oracle(v):
    """scale = rstd * gamma, shift = beta - mean * scale per (sample, channel); NULL gamma and
    beta read as 1 and 0."""
    import torch
    n, c, groups = 2, 96, 8
    mean = vae_synth.normal((n, groups), [125, 0], scale=2.0)
    rstd = np.abs(vae_synth.normal((n, groups), [125, 1])) + 0.1
    gamma = vae_synth.normal((c,), [125, 2], mean=1.0, scale=0.3)
    beta = vae_synth.normal((c,), [125, 3], scale=0.2)
    mr = torch.as_tensor(np.stack([mean, rstd], -1), dtype=torch.float32, device="cuda")
    for gm, bt in ((gamma, beta), (None, None)):
        ab = torch.empty((n, c, 2), dtype=torch.float32, device="cuda")
        v.vae_groupnorm_scale_shift(
            mr, c, groups, None if gm is None else torch.as_tensor(gm, device="cuda"),
            None if bt is None else torch.as_tensor(bt, device="cuda"), ab)
        torch.cuda.synchronize()
        got = ab.cpu().numpy().astype(np.float64)
        g = np.repeat(np.arange(groups), c // groups)
        m32 = mean.astype(np.float32).astype(np.float64)[:, g]
        r32 = rstd.astype(np.float32).astype(np.float64)[:, g]
        sc = r32 * (1.0 if gm is None else gm[None, :])
        shf = (0.0 if bt is None else bt[None, :]) - m32 * sc
        np.testing.assert_allclose(got[..., 0], sc, rtol=1e-6)
        np.testing.assert_allclose(got[..., 1], shf, rtol=1e-5, atol=1e-6)
