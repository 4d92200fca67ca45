"""Pins of the oracle's layers against brute force, torch CPU library routines, closed forms and
invariants. No GPU."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import vae_synth


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ------------------------------------------------------------------------------------------------
# Causal Conv3d
# ------------------------------------------------------------------------------------------------

def _brute_conv(x, w, b):
    """Seven nested loops with the causal/zero-pad index rules spelled out."""
    n_, t_, h_, w_, c_ = x.shape
    o_ = w.shape[0]
    y = np.zeros((n_, t_, h_, w_, o_))
    for n in range(n_):
        for t in range(t_):
            for h in range(h_):
                for ww in range(w_):
                    for o in range(o_):
                        s = b[o]
                        for c in range(c_):
                            for a in range(3):
                                ti = max(t + a - 2, 0)          # two replicated first frames
                                for p in range(3):
                                    hi = h + p - 1
                                    if hi < 0 or hi >= h_:
                                        continue                # zero padding
                                    for q in range(3):
                                        wi = ww + q - 1
                                        if wi < 0 or wi >= w_:
                                            continue
                                        s += w[o, c, a, p, q] * x[n, ti, hi, wi, c]
                        y[n, t, h, ww, o] = s
    return y


@pytest.mark.parametrize("shape", [(1, 3, 4, 5, 2), (2, 1, 3, 2, 3), (1, 4, 1, 1, 2)])
def test_conv_brute_force(shape):
    x = _rand(shape, 1)
    w = _rand((3, shape[-1], 3, 3, 3), 2)
    b = _rand((3,), 3)
    got = oracle.causal_conv3d(x, w, b)
    ref = _brute_conv(x, w, b)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_conv_matches_torch():
    x = _rand((2, 5, 7, 6, 4), 4)
    w = _rand((5, 4, 3, 3, 3), 5)
    b = _rand((5,), 6)
    xt = torch.from_numpy(x).permute(0, 4, 1, 2, 3)                    # NCDHW
    xt = torch.cat([xt[:, :, :1], xt[:, :, :1], xt], dim=2)            # causal replicate pad
    xt = F.pad(xt, (1, 1, 1, 1, 0, 0))                                 # zeros in H, W
    ref = F.conv3d(xt, torch.from_numpy(w), torch.from_numpy(b)).permute(0, 2, 3, 4, 1).numpy()
    np.testing.assert_allclose(oracle.causal_conv3d(x, w, b), ref, rtol=0, atol=1e-11)


def test_conv_is_causal():
    x = _rand((1, 6, 5, 5, 3), 7)
    w = _rand((2, 3, 3, 3, 3), 8)
    y0 = oracle.causal_conv3d(x, w)
    for tp in range(1, 6):
        x2 = x.copy()
        x2[:, tp] += 1.0
        y1 = oracle.causal_conv3d(x2, w)
        assert np.array_equal(y0[:, :tp], y1[:, :tp])
        assert not np.allclose(y0[:, tp], y1[:, tp])


def test_conv_time_constant_input_gives_time_constant_output():
    frame = _rand((1, 1, 4, 6, 3), 9)
    x = np.repeat(frame, 5, axis=1)
    y = oracle.causal_conv3d(x, _rand((2, 3, 3, 3, 3), 10), _rand((2,), 11))
    for t in range(1, 5):
        np.testing.assert_allclose(y[:, t], y[:, 0], rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# GroupNorm, statistics, SiLU
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("groups,c", [(8, 32), (32, 128), (32, 32), (4, 12)])
def test_group_norm_matches_torch(groups, c):
    x = _rand((2, 3, 4, 5, c), 12) * 2.0 + 0.5
    gamma, beta = _rand((c,), 13), _rand((c,), 14)
    ref = F.group_norm(torch.from_numpy(x).permute(0, 4, 1, 2, 3), groups,
                       torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-6)
    ref = ref.permute(0, 2, 3, 4, 1).numpy()
    np.testing.assert_allclose(oracle.group_norm(x, groups, 1e-6, gamma, beta), ref,
                               rtol=0, atol=1e-10)


def test_group_norm_closed_form():
    groups, eps = 4, 1e-3
    x = _rand((1, 2, 3, 4, 8), 15) * 3.0 + 7.0
    y = oracle.group_norm(x, groups, eps)
    xg = x.reshape(1, -1, groups, 2)
    yg = y.reshape(1, -1, groups, 2)
    for g in range(groups):
        s2 = xg[:, :, g].var()                  # biased variance of the group
        assert abs(yg[:, :, g].mean()) < 1e-12
        np.testing.assert_allclose(yg[:, :, g].var(), s2 / (s2 + eps), rtol=1e-12)


def _split_hw(x, hcuts, wcuts):
    hs = np.split(x, hcuts, axis=2)
    return [p for row in hs for p in np.split(row, wcuts, axis=3)]


@pytest.mark.parametrize("hcuts,wcuts", [([3], [1, 6]), ([1, 2, 6], [5]), ([], [2])])
def test_chan_combine_equals_whole(hcuts, wcuts):
    x = _rand((2, 3, 7, 8, 16), 16) + np.linspace(-3, 3, 8)[None, None, None, :, None]
    whole = oracle.group_moments(x, 4)
    n, mean, m2 = oracle.chan_combine(oracle.group_moments(p, 4) for p in _split_hw(x, hcuts, wcuts))
    assert np.array_equal(n, whole[0])
    np.testing.assert_allclose(mean, whole[1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(m2, whole[2], rtol=1e-12)


def _wrong_patch_gn(parts, groups, eps):
    """Per-patch mean and Bessel-corrected variance: the defect the DistVAE PatchGroupNorm fix
    removed. Used as a negative control only."""
    out = []
    for p in parts:
        pg = p.reshape(p.shape[0], -1, groups, p.shape[-1] // groups)
        mu = pg.mean(axis=(1, 3), keepdims=True)
        var = pg.var(axis=(1, 3), keepdims=True, ddof=1)
        out.append(((pg - mu) / np.sqrt(var + eps)).reshape(p.shape))
    return out


def test_negative_control_per_patch_bessel_fails():
    """The harness must reject the per-patch-mean + Bessel GroupNorm; Chan-merged stats pass."""
    x = _rand((1, 2, 6, 8, 16), 17)
    x[:, :, :, 4:] += 0.75                       # the right half is brighter
    parts = _split_hw(x, [], [4])
    whole = oracle.group_norm(x, 4, 1e-6)
    wrong = np.concatenate(_wrong_patch_gn(parts, 4, 1e-6), axis=3)
    rel_wrong = np.abs(wrong - whole).max() / np.abs(whole).max()
    assert rel_wrong > 1e-2
    n, mean, m2 = oracle.chan_combine(oracle.group_moments(p, 4) for p in parts)
    right = np.concatenate([oracle.normalize_with(p, 4, mean, m2 / n, 1e-6) for p in parts], axis=3)
    assert np.abs(right - whole).max() / np.abs(whole).max() < 1e-12


def test_large_mean_stress():
    """Mean 1e3, std 1: the hard case for variance maths that random weights never reach."""
    x = _rand((1, 4, 6, 10, 32), 18) + 1e3
    ref = F.group_norm(torch.from_numpy(x).permute(0, 4, 1, 2, 3), 8, eps=1e-6)
    ref = ref.permute(0, 2, 3, 4, 1).numpy()
    # torch's CPU kernel loses about 1e-9 here (its variance is not two-pass); ours is two-pass
    np.testing.assert_allclose(oracle.group_norm(x, 8, 1e-6), ref, rtol=0, atol=1e-8)
    n, mean, m2 = oracle.chan_combine(oracle.group_moments(p, 8) for p in _split_hw(x, [2], [3, 7]))
    whole = oracle.group_moments(x, 8)
    np.testing.assert_allclose(m2 / n, whole[2] / whole[0], rtol=1e-9)


def test_silu_identities():
    x = np.linspace(-30, 30, 601)
    s = oracle.silu(x)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - oracle.silu(-x), x, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(oracle.silu(np.array([-1e4, 1e4]))))
    np.testing.assert_allclose(s, x * torch.sigmoid(torch.from_numpy(x)).numpy(), atol=1e-14)


# ------------------------------------------------------------------------------------------------
# Upsampling
# ------------------------------------------------------------------------------------------------

def test_nearest_by_index():
    x = _rand((1, 2, 3, 4, 5), 19)
    y = oracle.nearest_upsample(x, 2, 3)
    assert y.shape == (1, 2, 6, 12, 5)
    for h in range(6):
        for w in range(12):
            assert np.array_equal(y[:, :, h, w], x[:, :, h // 2, w // 3])


@pytest.mark.parametrize("st,sh,sw", [(2, 2, 2), (1, 4, 4), (2, 1, 1), (1, 2, 3)])
def test_depth_to_space_by_index(st, sh, sw):
    c = 3
    x = _rand((1, 3, 2, 2, c * st * sh * sw), 20)
    y = oracle.depth_to_space(x, st, sh, sw)
    t_out = st * 3 - (st - 1)
    assert y.shape == (1, t_out, 2 * sh, 2 * sw, c)
    for to in range(t_out):
        tf = to + st - 1                        # frame index before the causal drop
        t, dt = divmod(tf, st)
        for ho in range(2 * sh):
            h, dh = divmod(ho, sh)
            for wo in range(2 * sw):
                w, dw = divmod(wo, sw)
                k = ((dt * sh + dh) * sw + dw) * c
                assert np.array_equal(y[0, to, ho, wo], x[0, t, h, w, k:k + c])


def test_depth_to_space_inverts_space_to_depth():
    x = _rand((1, 2, 4, 6, 5), 21)
    # space-to-depth written independently: gather each 2x3 block into channels
    s2d = np.concatenate([x[:, :, dh::2, dw::3] for dh in range(2) for dw in range(3)], axis=-1)
    np.testing.assert_array_equal(oracle.depth_to_space(s2d, 1, 2, 3), x)


def test_synth_bf16_rounding():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], dtype=np.float32)
    r = vae_synth.round_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0                      # tie -> even
    assert r[2] == np.float32(1.0 + 2 ** -6)                # tie -> even (up)
    assert r[3] == -2.5
    t = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(r, t)


# ------------------------------------------------------------------------------------------------
# RMS norm and frame attention (Wan-shaped decoder)
# ------------------------------------------------------------------------------------------------

def test_rms_norm_matches_torch_and_closed_form():
    import torch
    x = vae_synth.normal((2, 3, 4, 5, 64), [40, 1], scale=2.0, mean=0.5).astype(np.float64)
    gamma = vae_synth.normal((64,), [40, 2], scale=0.2, mean=1.0).astype(np.float64)
    beta = vae_synth.normal((64,), [40, 3], scale=0.1).astype(np.float64)
    got = oracle.rms_norm(x, 1e-6, gamma, beta)
    ref = torch.nn.functional.rms_norm(torch.as_tensor(x), (64,), torch.as_tensor(gamma),
                                       eps=1e-6).numpy() + beta
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # closed form: without the affine, the mean square over channels is ms / (ms + eps)
    y = oracle.rms_norm(x, 1e-3)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-3), rtol=1e-12)
    # positive scale invariance (eps = 0), and each position on its own
    np.testing.assert_allclose(oracle.rms_norm(3.5 * x, 0.0), oracle.rms_norm(x, 0.0), rtol=1e-12)
    np.testing.assert_allclose(oracle.rms_norm(x[:, :1], 1e-6), oracle.rms_norm(x, 1e-6)[:, :1],
                               rtol=0, atol=0)


def _attn_inputs(c, seed):
    g = vae_synth.normal((c,), [41, seed, 0], scale=0.2, mean=1.0).astype(np.float64)
    b = vae_synth.normal((c,), [41, seed, 1], scale=0.1).astype(np.float64)
    wq = vae_synth.normal((3 * c, c), [41, seed, 2], scale=1 / np.sqrt(c)).astype(np.float64)
    bq = vae_synth.normal((3 * c,), [41, seed, 3], scale=0.1).astype(np.float64)
    wo = vae_synth.normal((c, c), [41, seed, 4], scale=1 / np.sqrt(c)).astype(np.float64)
    bo = vae_synth.normal((c,), [41, seed, 5], scale=0.1).astype(np.float64)
    return g, b, wq, bq, wo, bo


def test_frame_attention_matches_torch_sdpa():
    import torch
    F = torch.nn.functional
    c = 32
    x = vae_synth.normal((2, 3, 4, 5, c), [42, 0]).astype(np.float64)
    g, b, wq, bq, wo, bo = _attn_inputs(c, 0)
    got = oracle.frame_attention(x, 1e-6, g, b, wq, bq, wo, bo)
    t = torch.as_tensor
    xt = t(x)
    xn = F.rms_norm(xt, (c,), t(g), eps=1e-6) + t(b)
    qkv = F.linear(xn.reshape(2, 3, 20, c), t(wq), t(bq))
    q, k, v = qkv[..., :c], qkv[..., c:2 * c], qkv[..., 2 * c:]
    o = F.scaled_dot_product_attention(q, k, v)            # softmax(q k^T / sqrt(c)) v
    ref = (F.linear(o, t(wo), t(bo)).reshape(x.shape) + xt).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_frame_attention_invariants():
    c = 16
    x = vae_synth.normal((1, 2, 3, 4, c), [43, 0]).astype(np.float64)
    g, b, wq, bq, wo, bo = _attn_inputs(c, 1)
    # zero queries: every position attends uniformly, so it receives the frame mean of v
    wq0, bq0 = wq.copy(), bq.copy()
    wq0[:c] = 0.0
    bq0[:c] = 0.0
    y = oracle.frame_attention(x, 1e-6, g, b, wq0, bq0, wo, bo)
    xn = oracle.rms_norm(x, 1e-6, g, b)
    v = xn @ wq[2 * c:].T + bq[2 * c:]
    vmean = v.mean(axis=(2, 3), keepdims=True)
    np.testing.assert_allclose(y, np.broadcast_to(vmean @ wo.T + bo, x.shape) + x, rtol=1e-12,
                               atol=1e-12)
    # permuting the positions of a frame permutes the output the same way
    y = oracle.frame_attention(x, 1e-6, g, b, wq, bq, wo, bo)
    perm = vae_synth.normal((12,), [43, 1]).argsort()
    xp = x.reshape(1, 2, 12, c)[:, :, perm].reshape(x.shape)
    yp = oracle.frame_attention(xp, 1e-6, g, b, wq, bq, wo, bo)
    np.testing.assert_allclose(yp.reshape(1, 2, 12, c), y.reshape(1, 2, 12, c)[:, :, perm],
                               rtol=1e-12, atol=1e-12)
    # frames do not see each other
    y1 = oracle.frame_attention(x[:, 1:], 1e-6, g, b, wq, bq, wo, bo)
    np.testing.assert_allclose(y1, y[:, 1:], rtol=0, atol=1e-14)


def test_attention_needs_the_whole_frame():
    """Negative control: attention applied per width patch differs from whole-frame attention."""
    c = 16
    x = vae_synth.normal((1, 1, 4, 6, c), [44, 0]).astype(np.float64)
    g, b, wq, bq, wo, bo = _attn_inputs(c, 2)
    whole = oracle.frame_attention(x, 1e-6, g, b, wq, bq, wo, bo)
    per_patch = np.concatenate([oracle.frame_attention(x[:, :, :, s], 1e-6, g, b, wq, bq, wo, bo)
                                for s in (slice(0, 3), slice(3, 6))], axis=3)
    assert np.abs(per_patch - whole).max() > 1e-2
