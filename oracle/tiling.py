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

Output boxes. A spatial span of latent rows [s, s + n) maps to output rows [s * r, (s + n) * r).
The temporal axis is causal: a clip of n latent frames decodes to 1 + (n - 1) * r frames, because
its first latent frame yields a single frame. The pages cut overlap tiles in time as well as in
space ("[TRTLLM-14029][feat] LTX-2 tile-parallel VAE decode", Approach: overlapping
spatial/temporal tiles), but say nothing of how a temporal tile's frames line up with the whole
video. The plainest reading that the causal decoder supports: a temporal tile of latent frames
[s, s + n), decoded alone, gives output frames [s * r, (s + n - 1) * r + 1). Its single first
frame takes the place of the last frame of latent frame s in the whole decode, and the frames of
each later latent frame line up with the whole decode's. For that reason consecutive temporal
tiles must share at least one latent frame when r > 1; otherwise the r - 1 frames before a
tile's first frame would come from no tile. Overlaps are measured between the output spans of
neighbouring tiles.
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


def out_span(start: int, size: int, scale: int, causal: bool):
    """Output span [lo, hi) of the latent span [start, start + size) along one axis."""
    if causal:
        return start * scale, (start + size - 1) * scale + 1
    return start * scale, (start + size) * scale


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


def _overlaps(outs):
    """Per tile along one axis: (lead, trail) overlap of its output span with the neighbours'."""
    lead, trail = [], []
    for k, (lo, hi) in enumerate(outs):
        lead.append(max(0, outs[k - 1][1] - lo) if k > 0 else 0)
        trail.append(max(0, hi - outs[k + 1][0]) if k + 1 < len(outs) else 0)
    return lead, trail


def overlap_tiles(t: int, h: int, w: int, tile_hw, stride_hw, scale, tile_t: int = 0,
                  stride_t: int = 0):
    """Overlapping tile list (row-major over T, H, W) with latent/output boxes and overlaps.

    ``tile_t`` <= 0 leaves the temporal axis whole."""
    st, sh, sw = scale
    ts = axis_tiles(t, tile_t, stride_t)
    if len(ts) > 1 and st > 1 and stride_t >= tile_t:
        raise ValueError(f"temporal stride {stride_t} must be below the tile ({tile_t}): "
                         "a causal tile's first frame leaves a gap otherwise")
    hs = axis_tiles(h, tile_hw[0], stride_hw[0])
    ws = axis_tiles(w, tile_hw[1], stride_hw[1])
    to = [out_span(s, n, st, True) for s, n in ts]
    ho = [out_span(s, n, sh, False) for s, n in hs]
    wo = [out_span(s, n, sw, False) for s, n in ws]
    lt, tt = _overlaps(to)
    lh, th = _overlaps(ho)
    lw, tw = _overlaps(wo)
    tiles = []
    for k, (t0, tn) in enumerate(ts):
        for i, (h0, hn) in enumerate(hs):
            for j, (w0, wn) in enumerate(ws):
                tiles.append({
                    "slab": k, "row": i, "col": j,
                    "latent": (t0, t0 + tn, h0, h0 + hn, w0, w0 + wn),
                    "out": to[k] + ho[i] + wo[j],
                    "lead": (lt[k], lh[i], lw[j]), "trail": (tt[k], th[i], tw[j]),
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
    """Sum over the distinct tiles along ``axis`` (0 = T, 1 = H, 2 = W) of their 1-D ramps."""
    seen = {}
    for tl in tiles:
        lo, hi = tl["out"][2 * axis], tl["out"][2 * axis + 1]
        seen[(lo, hi)] = (tl["lead"][axis], tl["trail"][axis])
    s = np.zeros(length, dtype=np.float64)
    for (lo, hi), (ld, tr) in seen.items():
        s[lo:hi] += ramp_1d(hi - lo, ld, tr)
    return s
