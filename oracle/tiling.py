"""Oracle tile and patch geometry: integer index maths, plus the 1-D blend ramps.

Test infrastructure: only tests, the smoke check and the benchmark's CPU-baseline leg use it.

Two ways of cutting a decode, both described on the pages:
- Patches (mode A, patch-halo). The latent is cut into bands along H and W. Every convolution
  reads a one-row/column halo from the neighbouring patches, and GroupNorm uses statistics merged
  across patches, so the result equals the untiled decode. Band rule: with L rows over p parts,
  the first L % p parts get one row more ("Add tiled VAE parallelism & extended model support",
  Patchify commit message).
- Overlapping tiles (mode B, overlap-blend). The latent is cut into tiles of ``tile`` rows whose
  starts step by ``stride``: 0, s, 2s, ... < L. Each tile has size min(tile, L - start). An axis
  no longer than ``tile`` is left whole. With tile 512, stride 448, the pixel extent 576 gives
  tiles 512 and 128, and 256 is left untiled ("[Feature] Support VAE tiling parallel encode for
  LTX-2", review thread). Each tile is decoded alone and blended with separable linear ramps,
  normalised by the summed weights ("[TRTLLM-14029][feat] LTX-2 tile-parallel VAE decode",
  Approach).

Ramps (the plainest reading of "blend ... divide"). Two consecutive tiles on an axis overlap by
E output samples. Over the overlap, the later tile's leading weight is (j+1)/(E+1) and the earlier
tile's trailing weight is (E-j)/(E+1), for j = 0..E-1. Elsewhere the weight is 1, and a tile's
weight is the product over axes.

Output boxes: spatial output = latent x scale. The temporal axis is never split and maps T latent
frames to 1 + (T-1) * scale_t output frames (causal).
"""
from __future__ import annotations

import numpy as np


def bands(length: int, parts: int):
    """(start, size) of ``parts`` contiguous bands over ``length`` rows; larger bands first."""
    if parts < 1 or parts > length:
        raise ValueError(f"cannot cut {length} rows into {parts} non-empty bands")
    q, r = divmod(length, parts)
    out, start = [], 0
    for i in range(parts):
        size = q + 1 if i < r else q
        out.append((start, size))
        start += size
    return out


def axis_tiles(length: int, tile: int, stride: int):
    """(start, size) of the overlapping tiles along one axis."""
    if tile <= 0 or length <= tile:
        return [(0, length)]
    if stride <= 0 or stride > tile:
        raise ValueError(f"stride {stride} must be in 1..tile ({tile}) so tiles leave no gap")
    return [(s, min(tile, length - s)) for s in range(0, length, stride)]


def _out_t(t: int, scale_t: int) -> int:
    return 1 + (t - 1) * scale_t


def patch_tiles(t: int, h: int, w: int, ph: int, pw: int, scale):
    """Patch list (row-major) with latent and output boxes; overlaps are all zero."""
    st, sh, sw = scale
    tiles = []
    for i, (h0, hs) in enumerate(bands(h, ph)):
        for j, (w0, ws) in enumerate(bands(w, pw)):
            tiles.append({
                "row": i, "col": j,
                "latent": (0, t, h0, h0 + hs, w0, w0 + ws),
                "out": (0, _out_t(t, st), h0 * sh, (h0 + hs) * sh, w0 * sw, (w0 + ws) * sw),
                "lead": (0, 0, 0), "trail": (0, 0, 0),
            })
    return tiles


def _overlaps(spans, scale):
    """Per tile along one axis: (lead, trail) overlap with the neighbours, in output samples."""
    lead, trail = [], []
    for k, (s, n) in enumerate(spans):
        if k > 0:
            ps, pn = spans[k - 1]
            lead.append(max(0, ps + pn - s) * scale)
        else:
            lead.append(0)
        if k + 1 < len(spans):
            ns, _ = spans[k + 1]
            trail.append(max(0, s + n - ns) * scale)
        else:
            trail.append(0)
    return lead, trail


def overlap_tiles(t: int, h: int, w: int, tile_hw, stride_hw, scale):
    """Overlapping tile list (row-major over H then W) with latent/output boxes and overlaps."""
    st, sh, sw = scale
    hs = axis_tiles(h, tile_hw[0], stride_hw[0])
    ws = axis_tiles(w, tile_hw[1], stride_hw[1])
    lh, th = _overlaps(hs, sh)
    lw, tw = _overlaps(ws, sw)
    tiles = []
    for i, (h0, hn) in enumerate(hs):
        for j, (w0, wn) in enumerate(ws):
            tiles.append({
                "row": i, "col": j,
                "latent": (0, t, h0, h0 + hn, w0, w0 + wn),
                "out": (0, _out_t(t, st), h0 * sh, (h0 + hn) * sh, w0 * sw, (w0 + wn) * sw),
                "lead": (0, lh[i], lw[j]), "trail": (0, th[i], tw[j]),
            })
    return tiles


def ramp_1d(size: int, lead: int, trail: int) -> np.ndarray:
    """Blend weight along one axis of a tile of ``size`` output samples."""
    j = np.arange(size, dtype=np.float64)
    w = np.ones(size, dtype=np.float64)
    if lead > 0:
        m = j < lead
        w[m] *= (j[m] + 1.0) / (lead + 1.0)
    if trail > 0:
        m = (size - j) <= trail
        w[m] *= (size - j[m]) / (trail + 1.0)
    return w


def axis_weight_sum(tiles, axis: int, length: int) -> np.ndarray:
    """Sum over the distinct tiles along ``axis`` (1 = H, 2 = W) of their 1-D ramps."""
    seen = {}
    for tl in tiles:
        lo, hi = tl["out"][2 * axis], tl["out"][2 * axis + 1]
        seen[(lo, hi)] = (tl["lead"][axis], tl["trail"][axis])
    s = np.zeros(length, dtype=np.float64)
    for (lo, hi), (ld, tr) in seen.items():
        s[lo:hi] += ramp_1d(hi - lo, ld, tr)
    return s
