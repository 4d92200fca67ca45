"""Oracle decoders: whole, patch-halo (mode A) and overlap-blend (mode B). Channels-last, float64.

Test infrastructure: only tests, the smoke check and the benchmark's CPU-baseline leg use it.

The layer plan and parameters come from ``vae_synth``: a list of ops and a parameter list in plan
order. A residual block is GN+SiLU, conv, GN+SiLU, conv, plus its input; ``res_rms`` is the same
block with RMS norms, ``rms_silu`` an RMS norm followed by SiLU, and ``attn`` the single-head
frame attention block (``layers.frame_attention``).

``decode_patch_halo`` deliberately does not call ``decode``. It is the patch-sharded computation of
"Add tiled VAE parallelism & extended model support" (PatchConv3d / PatchGroupNorm commit messages):
- every patch keeps its own activation;
- a convolution gathers a one-row/column halo from the neighbouring patches and pads zeros only
  where the patch meets the true image border;
- GroupNorm merges per-patch (count, mean, M2) with Chan's formula before normalising.
It must reproduce the whole decode, which tests pin.

``decode_overlap_blend`` is the serial tiled decode of "[TRTLLM-14029][feat] LTX-2 tile-parallel VAE
decode" (Description and Approach). Each tile is decoded on its own with its own borders and
GroupNorm statistics. The tile is then blended into a full-size buffer, its weights go into a weight
buffer, and the buffer is divided by the weights at the end.
"""
from __future__ import annotations

import numpy as np

from .layers import causal_conv3d, causal_time_pad, conv3d_valid, group_norm, silu, \
    nearest_upsample, depth_to_space, space_to_depth, rms_norm, frame_attention, \
    strided_causal_conv3d

# Spatial zero padding of a strided downsampling conv ("conv_down"), ((top, bottom), (left,
# right)): one row and column on every side (LTX-2's bare strided conv), or none before and one
# after (Wan's downsampler pads (0, 1, 0, 1) before striding). "Add tiled VAE parallelism &
# extended model support", LTX-2 and Qwen-Image/Wan encoder commit messages.
DOWN_PADS = {"around": ((1, 1), (1, 1)), "after": ((0, 1), (0, 1))}
from .stats import group_moments, chan_combine, normalize_with
from .tiling import bands, overlap_tiles, ramp_1d


def output_shape(spec: dict, latent_shape):
    """[N, T, H, W, C] of the decoder output for an NDHWC latent shape, following the plan."""
    n, t, h, w, c = latent_shape
    for op in spec["layers"]:
        k = op["op"]
        if k == "conv":
            c = op["cout"]
        elif k == "d2s":
            st, sh, sw = op["st"], op["sh"], op["sw"]
            t, h, w, c = st * t - (st - 1), h * sh, w * sw, c // (st * sh * sw)
        elif k == "nearest":
            h, w = h * op["sh"], w * op["sw"]
        elif k == "s2d":
            st, sh, sw = op["st"], op["sh"], op["sw"]
            t, h, w, c = (t + st - 1) // st, h // sh, w // sw, c * st * sh * sw
        elif k == "conv_down":
            (pt, pb), (pl, pr) = DOWN_PADS[op["pad"]]
            t = (t - 1) // op["st"] + 1
            h = (h + pt + pb - 3) // op["sh"] + 1
            w = (w + pl + pr - 3) // op["sw"] + 1
            c = op["cout"]
    return (n, t, h, w, c)


# ------------------------------------------------------------------------------------------------
# Whole decode
# ------------------------------------------------------------------------------------------------

def decode(spec: dict, z: np.ndarray, params: list) -> np.ndarray:
    """Untiled decode of the NDHWC latent ``z``; returns the NDHWC float64 output."""
    groups, eps = spec["groups"], spec["eps"]
    it = iter(params)
    h = np.asarray(z, dtype=np.float64)
    for op in spec["layers"]:
        k = op["op"]
        if k == "conv":
            p = next(it)
            h = causal_conv3d(h, p["w"], p["b"])
        elif k == "res":
            g1, c1, g2, c2 = next(it), next(it), next(it), next(it)
            t = silu(group_norm(h, groups, eps, g1["gamma"], g1["beta"]))
            t = causal_conv3d(t, c1["w"], c1["b"])
            t = silu(group_norm(t, groups, eps, g2["gamma"], g2["beta"]))
            h = causal_conv3d(t, c2["w"], c2["b"]) + h
            del t
        elif k == "gn_silu":
            g = next(it)
            h = silu(group_norm(h, groups, eps, g["gamma"], g["beta"]))
        elif k == "res_rms":
            g1, c1, g2, c2 = next(it), next(it), next(it), next(it)
            t = silu(rms_norm(h, eps, g1["gamma"], g1["beta"]))
            t = causal_conv3d(t, c1["w"], c1["b"])
            t = silu(rms_norm(t, eps, g2["gamma"], g2["beta"]))
            h = causal_conv3d(t, c2["w"], c2["b"]) + h
            del t
        elif k == "rms_silu":
            g = next(it)
            h = silu(rms_norm(h, eps, g["gamma"], g["beta"]))
        elif k == "attn":
            a = next(it)
            h = frame_attention(h, eps, a["gamma"], a["beta"], a["w_qkv"], a["b_qkv"], a["w_out"],
                                a["b_out"])
        elif k == "d2s":
            h = depth_to_space(h, op["st"], op["sh"], op["sw"])
        elif k == "nearest":
            h = nearest_upsample(h, op["sh"], op["sw"])
        elif k == "s2d":
            h = space_to_depth(h, op["st"], op["sh"], op["sw"])
        elif k == "conv_down":
            p = next(it)
            h = strided_causal_conv3d(h, p["w"], p["b"], (op["st"], op["sh"], op["sw"]),
                                      DOWN_PADS[op["pad"]])
        else:
            raise ValueError(k)
    return h


def decode_causal_clips(spec: dict, z: np.ndarray, params: list, clip: int) -> np.ndarray:
    """Decode clip by clip: latent frames [0, clip), [clip, 2 clip), ... one after another, each
    clip seeing only its own frames plus what the clips before it left behind.

    Every causal conv keeps the last two frames of its input (its temporal receptive field beyond
    the current frame) and puts them in front of the next clip's input instead of the causal copies
    of frame 0, which only the first clip gets. A causal depth-to-space drops its leading frames
    in the first clip only. This is the plainest reading of the tile-parallel decode's temporal
    tiles with the causal context carried ("[TRTLLM-14029][feat] LTX-2 tile-parallel VAE decode",
    Description: overlapping spatial/temporal tiles of a causal decoder): carried, not
    overlapped, the clips rebuild the whole decode exactly. That holds only for plans whose every
    op is local in time; a GroupNorm's statistics span all frames, so such plans are refused.
    """
    kinds = {op["op"] for op in spec["layers"]}
    assert not kinds & {"res", "gn_silu", "s2d", "conv_down"}, \
        f"clip-by-clip decode needs ops local in time, not {sorted(kinds)}"
    z = np.asarray(z, dtype=np.float64)
    eps = spec["eps"]
    caches = {}

    def conv(h, p, key):
        prev = caches.get(key)
        if prev is None:
            prev = np.concatenate([h[:, :1]] * 2, axis=1)       # causal copies of frame 0
        ext = np.concatenate([prev, h], axis=1)
        caches[key] = ext[:, -2:]
        ext = np.pad(ext, ((0, 0), (0, 0), (1, 1), (1, 1), (0, 0)))
        return conv3d_valid(ext, p["w"], p["b"])

    outs = []
    for c0 in range(0, z.shape[1], clip):
        h = z[:, c0:c0 + clip]
        it = iter(params)
        for i, op in enumerate(spec["layers"]):
            k = op["op"]
            if k == "conv":
                h = conv(h, next(it), (i, 0))
            elif k == "res_rms":
                g1, c1, g2, c2 = next(it), next(it), next(it), next(it)
                t = conv(silu(rms_norm(h, eps, g1["gamma"], g1["beta"])), c1, (i, 1))
                t = silu(rms_norm(t, eps, g2["gamma"], g2["beta"]))
                h = conv(t, c2, (i, 2)) + h
            elif k == "rms_silu":
                g = next(it)
                h = silu(rms_norm(h, eps, g["gamma"], g["beta"]))
            elif k == "attn":
                a = next(it)
                h = frame_attention(h, eps, a["gamma"], a["beta"], a["w_qkv"], a["b_qkv"],
                                    a["w_out"], a["b_out"])
            elif k == "d2s":
                h = depth_to_space(h, op["st"], op["sh"], op["sw"], drop=c0 == 0)
            elif k == "nearest":
                h = nearest_upsample(h, op["sh"], op["sw"])
            else:
                raise ValueError(k)
        outs.append(h)
    return np.concatenate(outs, axis=1)


def encode(spec: dict, x: np.ndarray, params: list) -> np.ndarray:
    """Untiled encode of the NDHWC video ``x``: the same plan executor as ``decode``; an encoder
    plan narrows with ``s2d`` folds where a decoder widens with ``d2s``."""
    return decode(spec, x, params)


# ------------------------------------------------------------------------------------------------
# Mode A: patch-halo decode
# ------------------------------------------------------------------------------------------------

def _starts(sizes):
    return [int(s) for s in np.concatenate([[0], np.cumsum(sizes)[:-1]])]


def _conv_patches(patches, w, b):
    """Convolve every patch with a one-row/column halo gathered from the other patches."""
    rows = [row[0].shape[2] for row in patches]
    cols = [p.shape[3] for p in patches[0]]
    r_at, c_at = _starts(rows), _starts(cols)
    n, t, _, _, c = patches[0][0].shape
    out = []
    for i in range(len(rows)):
        out_row = []
        for j in range(len(cols)):
            r0, r1 = r_at[i] - 1, r_at[i] + rows[i] + 1     # halo-extended region
            c0, c1 = c_at[j] - 1, c_at[j] + cols[j] + 1
            ext = np.zeros((n, t, r1 - r0, c1 - c0, c))    # outside the image: zero padding
            for a in range(len(rows)):
                lo_r, hi_r = max(r0, r_at[a]), min(r1, r_at[a] + rows[a])
                if lo_r >= hi_r:
                    continue
                for bb in range(len(cols)):
                    lo_c, hi_c = max(c0, c_at[bb]), min(c1, c_at[bb] + cols[bb])
                    if lo_c >= hi_c:
                        continue
                    ext[:, :, lo_r - r0:hi_r - r0, lo_c - c0:hi_c - c0] = \
                        patches[a][bb][:, :, lo_r - r_at[a]:hi_r - r_at[a],
                                       lo_c - c_at[bb]:hi_c - c_at[bb]]
            y = conv3d_valid(causal_time_pad(ext, 3), w, b)
            # a convolved patch keeps the size of the patch it came from
            assert y.shape[2:4] == (rows[i], cols[j]), (y.shape, rows[i], cols[j])
            out_row.append(y)
        out.append(out_row)
    return out


def _conv_down_patches(patches, w, b, stride, pads):
    """Strided conv of every patch. A patch's output rows [a / s, (a + n) / s) read input rows
    s * o - top + (0, 1, 2): its own band plus `top` rows gathered before it and `bottom` after
    (for a band of whole strides); zeros only beyond the true image border. The gathered region is
    then convolved without further padding."""
    (pt, pb), (pl, pr) = pads
    rows = [row[0].shape[2] for row in patches]
    cols = [p.shape[3] for p in patches[0]]
    r_at, c_at = _starts(rows), _starts(cols)
    n, t, _, _, c = patches[0][0].shape
    out = []
    for i in range(len(rows)):
        out_row = []
        for j in range(len(cols)):
            assert rows[i] % stride[1] == 0 and cols[j] % stride[2] == 0, (rows, cols, stride)
            r0, r1 = r_at[i] - pt, r_at[i] + rows[i] + pb
            c0, c1 = c_at[j] - pl, c_at[j] + cols[j] + pr
            ext = np.zeros((n, t, r1 - r0, c1 - c0, c))
            for a in range(len(rows)):
                lo_r, hi_r = max(r0, r_at[a]), min(r1, r_at[a] + rows[a])
                if lo_r >= hi_r:
                    continue
                for bb in range(len(cols)):
                    lo_c, hi_c = max(c0, c_at[bb]), min(c1, c_at[bb] + cols[bb])
                    if lo_c >= hi_c:
                        continue
                    ext[:, :, lo_r - r0:hi_r - r0, lo_c - c0:hi_c - c0] = \
                        patches[a][bb][:, :, lo_r - r_at[a]:hi_r - r_at[a],
                                       lo_c - c_at[bb]:hi_c - c_at[bb]]
            y = strided_causal_conv3d(ext, w, b, stride, ((0, 0), (0, 0)))
            assert y.shape[2:4] == (rows[i] // stride[1], cols[j] // stride[2]), y.shape
            out_row.append(y)
        out.append(out_row)
    return out


def _gn_patches(patches, groups, eps, gamma, beta, act):
    """GroupNorm over the union of all patches via per-patch moments merged with Chan's formula."""
    parts = [group_moments(p, groups) for row in patches for p in row]   # owned positions only
    n, mean, m2 = chan_combine(parts)
    var = m2 / n                                                          # biased
    out = [[normalize_with(p, groups, mean, var, eps, gamma, beta) for p in row] for row in patches]
    if act:
        out = [[silu(p) for p in row] for row in out]
    return out


def decode_patch_halo(spec: dict, z: np.ndarray, params: list, grid, unit=(1, 1)) -> np.ndarray:
    """Decode with the latent cut into ph x pw patches (bands along H and W).

    ``unit``: the bands are cut in whole multiples of it (rows, columns). An encoder plan folds
    space into channels, so its bands must be multiples of the total fold ("Add tiled VAE
    parallelism & extended model support", encoder commit: bands in whole multiples of what the
    VAE narrows the axis by, the first ranks taking one band more)."""
    ph, pw = grid
    groups, eps = spec["groups"], spec["eps"]
    z = np.asarray(z, dtype=np.float64)
    uh, uw = unit
    assert z.shape[2] % uh == 0 and z.shape[3] % uw == 0, (z.shape, unit)
    hb = [(s * uh, n * uh) for s, n in bands(z.shape[2] // uh, ph)]
    wb = [(s * uw, n * uw) for s, n in bands(z.shape[3] // uw, pw)]
    patches = [[z[:, :, h0:h0 + hs, w0:w0 + ws] for (w0, ws) in wb] for (h0, hs) in hb]
    it = iter(params)
    for op in spec["layers"]:
        k = op["op"]
        if k == "conv":
            p = next(it)
            patches = _conv_patches(patches, p["w"], p["b"])
        elif k == "res":
            g1, c1, g2, c2 = next(it), next(it), next(it), next(it)
            t = _gn_patches(patches, groups, eps, g1["gamma"], g1["beta"], True)
            t = _conv_patches(t, c1["w"], c1["b"])
            t = _gn_patches(t, groups, eps, g2["gamma"], g2["beta"], True)
            t = _conv_patches(t, c2["w"], c2["b"])
            patches = [[a + bb for a, bb in zip(ra, rb)] for ra, rb in zip(t, patches)]
        elif k == "gn_silu":
            g = next(it)
            patches = _gn_patches(patches, groups, eps, g["gamma"], g["beta"], True)
        elif k == "res_rms":
            # RMS norms reduce over channels: each patch normalises its own positions
            g1, c1, g2, c2 = next(it), next(it), next(it), next(it)
            t = [[silu(rms_norm(p, eps, g1["gamma"], g1["beta"])) for p in row] for row in patches]
            t = _conv_patches(t, c1["w"], c1["b"])
            t = [[silu(rms_norm(p, eps, g2["gamma"], g2["beta"])) for p in row] for row in t]
            t = _conv_patches(t, c2["w"], c2["b"])
            patches = [[a + bb for a, bb in zip(ra, rb)] for ra, rb in zip(t, patches)]
        elif k == "rms_silu":
            g = next(it)
            patches = [[silu(rms_norm(p, eps, g["gamma"], g["beta"])) for p in row]
                       for row in patches]
        elif k == "attn":
            # the frame is gathered whole around the attention, then cut back into the same bands
            a = next(it)
            rows = [row[0].shape[2] for row in patches]
            cols = [p.shape[3] for p in patches[0]]
            whole = np.concatenate([np.concatenate(row, axis=3) for row in patches], axis=2)
            whole = frame_attention(whole, eps, a["gamma"], a["beta"], a["w_qkv"], a["b_qkv"],
                                    a["w_out"], a["b_out"])
            r_at, c_at = _starts(rows), _starts(cols)
            patches = [[whole[:, :, r_at[i]:r_at[i] + rows[i], c_at[j]:c_at[j] + cols[j]]
                        for j in range(len(cols))] for i in range(len(rows))]
        elif k == "d2s":
            patches = [[depth_to_space(p, op["st"], op["sh"], op["sw"]) for p in row]
                       for row in patches]
        elif k == "nearest":
            patches = [[nearest_upsample(p, op["sh"], op["sw"]) for p in row] for row in patches]
        elif k == "s2d":
            # bands are cut in whole multiples of the fold, so every patch folds on its own
            patches = [[space_to_depth(p, op["st"], op["sh"], op["sw"]) for p in row]
                       for row in patches]
        elif k == "conv_down":
            p = next(it)
            patches = _conv_down_patches(patches, p["w"], p["b"], (op["st"], op["sh"], op["sw"]),
                                         DOWN_PADS[op["pad"]])
        else:
            raise ValueError(k)
    return np.concatenate([np.concatenate(row, axis=3) for row in patches], axis=2)


# ------------------------------------------------------------------------------------------------
# Mode B: overlap-blend decode
# ------------------------------------------------------------------------------------------------

def merge_tiles(tile_outputs, tiles, out_shape) -> np.ndarray:
    """Blend per-tile outputs into the full output: sum(w * y) / sum(w), weights accumulated."""
    acc = np.zeros(out_shape, dtype=np.float64)
    wsum = np.zeros(tuple(out_shape[:4]) + (1,), dtype=np.float64)
    for y, tl in zip(tile_outputs, tiles):
        t0, t1, h0, h1, w0, w1 = tl["out"]
        rt = ramp_1d(t1 - t0, tl["lead"][0], tl["trail"][0])
        rh = ramp_1d(h1 - h0, tl["lead"][1], tl["trail"][1])
        rw = ramp_1d(w1 - w0, tl["lead"][2], tl["trail"][2])
        wt = (rt[:, None, None] * rh[None, :, None] * rw[None, None, :])[None, ..., None]
        acc[:, t0:t1, h0:h1, w0:w1] += np.asarray(y, dtype=np.float64) * wt
        wsum[:, t0:t1, h0:h1, w0:w1] += wt
    return acc / wsum


def decode_overlap_blend(spec: dict, z: np.ndarray, params: list, tile_hw, stride_hw,
                         scale, tile_t: int = 0, stride_t: int = 0) -> np.ndarray:
    """Serial overlap-blend tiled decode of the NDHWC latent ``z`` (``tile_t`` > 0 also cuts T)."""
    z = np.asarray(z, dtype=np.float64)
    _, t, h, w, _ = z.shape
    tiles = overlap_tiles(t, h, w, tile_hw, stride_hw, scale, tile_t, stride_t)
    out_shape = output_shape(spec, z.shape)
    outs = []
    for tl in tiles:
        t0, t1, h0, h1, w0, w1 = tl["latent"]
        y = decode(spec, z[:, t0:t1, h0:h1, w0:w1], params)    # own borders, own statistics
        o = tl["out"]
        assert y.shape[1:4] == (o[1] - o[0], o[3] - o[2], o[5] - o[4]), (y.shape, o)
        outs.append(y)
    return merge_tiles(outs, tiles, out_shape)


# ------------------------------------------------------------------------------------------------
# Encode
# ------------------------------------------------------------------------------------------------

def encode_patch_halo(spec: dict, x: np.ndarray, params: list, grid) -> np.ndarray:
    """Patch-halo encode: bands in whole multiples of the plan's spatial fold (spec["down"])."""
    return decode_patch_halo(spec, x, params, grid, unit=tuple(spec["down"][1:]))


def encode_overlap_blend(spec: dict, x: np.ndarray, params: list, tile_hw, stride_hw) -> np.ndarray:
    """Serial overlap-blend tiled encode of the NDHWC video ``x``.

    The tile grid is cut on the latent grid (``tile_hw``, ``stride_hw`` in latent rows: 16 / 14 are
    512 / 448 pixels at a fold of 32, i.e. 64 pixels of overlap). Each tile encodes its pixel crop
    alone, with its own borders and statistics, T whole, and the latent tiles are blended with the
    same separable ramps as decoded tiles, in latent space ("[Feature] Support VAE tiling parallel
    encode for LTX-2", Purpose and review thread: sample tiles 512 with stride 448, per-tile latent
    shapes, a blend of the latents)."""
    x = np.asarray(x, dtype=np.float64)
    dt, dh, dw = spec["down"]
    out_shape = output_shape(spec, x.shape)
    _, lt, lh, lw, _ = out_shape
    assert x.shape[2] == lh * dh and x.shape[3] == lw * dw, (x.shape, out_shape)
    tiles = overlap_tiles(lt, lh, lw, tile_hw, stride_hw, (1, 1, 1))
    outs = []
    for tl in tiles:
        _, _, h0, h1, w0, w1 = tl["latent"]
        y = decode(spec, x[:, :, h0 * dh:h1 * dh, w0 * dw:w1 * dw], params)
        assert y.shape[1:4] == (lt, h1 - h0, w1 - w0), (y.shape, tl)
        outs.append(y)
    return merge_tiles(outs, tiles, out_shape)
