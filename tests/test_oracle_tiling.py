"""Pins of the oracle's tile and band geometry, blend ramps and merge. No GPU."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tile_grids.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_page_printed_axis_tiles():
    for case in _golden()["overlap_axes"]:
        got = oracle.axis_tiles(case["length"], case["tile"], case["stride"])
        assert [list(t) for t in got] == case["tiles"], case["cite"]


def test_page_printed_grid():
    for case in _golden()["overlap_grids"]:
        tiles = oracle.overlap_tiles(1, case["h"], case["w"], (case["tile"],) * 2,
                                     (case["stride"],) * 2, (1, 1, 1))
        sizes = [[t["latent"][3] - t["latent"][2], t["latent"][5] - t["latent"][4]] for t in tiles]
        assert sizes == case["sizes_hw"], case["cite"]


def test_page_printed_bands():
    for case in _golden()["bands"]:
        assert [s for _, s in oracle.bands(case["length"], case["parts"])] == case["sizes"], \
            case["cite"]


def test_latent_grid_of_the_720p_workload():
    # tile 512 px, stride 448 px at 32x spatial compression = 16 / 14 latent
    assert oracle.axis_tiles(22, 16, 14) == [(0, 16), (14, 8)]
    assert oracle.axis_tiles(40, 16, 14) == [(0, 16), (14, 16), (28, 12)]


@pytest.mark.parametrize("length,parts", [(40, 4), (22, 4), (7, 7), (17, 3), (1, 1), (100, 7)])
def test_band_rule(length, parts):
    b = oracle.bands(length, parts)
    sizes = [s for _, s in b]
    assert sum(sizes) == length
    assert max(sizes) - min(sizes) <= 1
    assert sizes == sorted(sizes, reverse=True)
    assert [s for s, _ in b] == list(np.cumsum([0] + sizes[:-1]))


def test_band_refusals():
    with pytest.raises(ValueError):
        oracle.bands(3, 4)
    with pytest.raises(ValueError):
        oracle.bands(3, 0)
    with pytest.raises(ValueError):
        oracle.axis_tiles(40, 8, 9)             # stride > tile would leave a gap


def test_patch_tiles_boxes():
    tiles = oracle.patch_tiles(16, 22, 40, 1, 4, (8, 32, 32))
    assert [t["latent"][4:] for t in tiles] == [(0, 10), (10, 20), (20, 30), (30, 40)]
    assert all(t["out"][:4] == (0, 121, 0, 704) for t in tiles)
    assert [t["out"][4:] for t in tiles] == [(0, 320), (320, 640), (640, 960), (960, 1280)]


def test_overlaps_and_ramps_sum_to_one():
    tiles = oracle.overlap_tiles(16, 22, 40, (16, 16), (14, 14), (8, 32, 32))
    assert len(tiles) == 6
    assert tiles[0]["trail"][1:] == (64, 64) and tiles[0]["lead"][1:] == (0, 0)
    assert tiles[4]["lead"][1:] == (64, 64)
    for axis, length in ((1, 704), (2, 1280)):
        s = oracle.axis_weight_sum(tiles, axis, length)
        np.testing.assert_allclose(s, 1.0, rtol=0, atol=1e-15)


def test_ramp_values():
    r = oracle.ramp_1d(6, 2, 3)
    np.testing.assert_allclose(r, [1 / 3, 2 / 3, 1, 3 / 4, 2 / 4, 1 / 4])
    assert np.all(oracle.ramp_1d(2, 2, 0) > 0)


def _crop_tiles(y, tiles):
    return [y[:, t["out"][0]:t["out"][1], t["out"][2]:t["out"][3], t["out"][4]:t["out"][5]]
            for t in tiles]


@pytest.mark.parametrize("grid", [((16, 16), (14, 14)), ((9, 9), (5, 5)), ((30, 30), (1, 1)),
                                  ((4, 5), (2, 5))])
def test_merge_of_exact_crops_is_identity(grid):
    tiles = oracle.overlap_tiles(3, 22, 17, grid[0], grid[1], (2, 1, 1))
    y = np.random.default_rng(0).standard_normal((1, 5, 22, 17, 3))
    merged = oracle.merge_tiles(_crop_tiles(y, tiles), tiles, y.shape)
    np.testing.assert_allclose(merged, y, rtol=1e-15, atol=1e-15)


def test_merge_preserves_constant_and_single_tile():
    tiles = oracle.overlap_tiles(2, 13, 11, (5, 4), (3, 3), (1, 2, 2))
    shape = (1, 2, 26, 22, 2)
    outs = [np.full((1, 2, t["out"][3] - t["out"][2], t["out"][5] - t["out"][4], 2), 2.5)
            for t in tiles]
    np.testing.assert_allclose(oracle.merge_tiles(outs, tiles, shape), 2.5, rtol=1e-15)
    one = oracle.overlap_tiles(2, 13, 11, (13, 11), (13, 11), (1, 2, 2))
    assert len(one) == 1
    y = np.random.default_rng(1).standard_normal(shape)
    assert np.array_equal(oracle.merge_tiles([y], one, shape), y)


# ------------------------------------------------------------------------------------------------
# Temporal tiles (overlap-blend). A clip of latent frames [s, s + n) decodes to output frames
# [s * r, (s + n - 1) * r + 1): its single first frame stands for the last frame of latent frame s.
# ------------------------------------------------------------------------------------------------

def test_temporal_grid_by_hand():
    # 16 latent frames, tiles of 8 stepping by 6, r = 8: clips [0,8), [6,14), [12,16) decode to
    # 57, 57 and 25 frames at output frames 0, 48 and 96; neighbours share 9 output frames.
    tiles = oracle.overlap_tiles(16, 22, 40, (0, 0), (0, 0), (8, 32, 32), 8, 6)
    assert [t["latent"][:2] for t in tiles] == [(0, 8), (6, 14), (12, 16)]
    assert [t["out"][:2] for t in tiles] == [(0, 57), (48, 105), (96, 121)]
    assert [t["lead"][0] for t in tiles] == [0, 9, 9]
    assert [t["trail"][0] for t in tiles] == [9, 9, 0]
    assert all(t["out"][2:] == (0, 704, 0, 1280) for t in tiles)
    np.testing.assert_allclose(oracle.axis_weight_sum(tiles, 0, 121), 1.0, rtol=0, atol=1e-15)


def test_temporal_tiles_are_t_major_and_cover_the_output():
    tiles = oracle.overlap_tiles(7, 22, 40, (16, 16), (14, 14), (4, 2, 2), 3, 2)
    assert len(tiles) == 4 * 2 * 3          # clip starts 0, 2, 4, 6
    assert [t["slab"] for t in tiles] == sorted(t["slab"] for t in tiles)
    covered = np.zeros(1 + 6 * 4, dtype=bool)
    for t in tiles:
        covered[t["out"][0]:t["out"][1]] = True
        assert t["out"][1] - t["out"][0] == 1 + (t["latent"][1] - t["latent"][0] - 1) * 4
    assert covered.all()
    assert np.all(oracle.axis_weight_sum(tiles, 0, 25) > 0)


def test_temporal_refusals():
    with pytest.raises(ValueError):        # r > 1: tiles that share no latent frame leave a gap
        oracle.overlap_tiles(16, 4, 4, (0, 0), (0, 0), (8, 1, 1), 8, 8)
    # r = 1 has no single first frame, so abutting clips are fine
    tiles = oracle.overlap_tiles(16, 4, 4, (0, 0), (0, 0), (1, 1, 1), 8, 8)
    assert [t["out"][:2] for t in tiles] == [(0, 8), (8, 16)]


@pytest.mark.parametrize("tt,stt", [(3, 2), (4, 2), (5, 1), (2, 1)])
def test_temporal_merge_of_exact_crops_is_identity(tt, stt):
    tiles = oracle.overlap_tiles(7, 9, 8, (5, 4), (3, 3), (4, 2, 2), tt, stt)
    y = np.random.default_rng(2).standard_normal((1, 25, 18, 16, 2))
    merged = oracle.merge_tiles(_crop_tiles(y, tiles), tiles, y.shape)
    np.testing.assert_allclose(merged, y, rtol=1e-15, atol=1e-15)


_LOCAL_PLAN = {
    # no convolution and no norm: every output frame depends on one latent frame only
    "groups": 1, "eps": 1e-6, "scale": (4, 2, 2),
    "layers": [{"op": "d2s", "st": 2, "sh": 2, "sw": 1},
               {"op": "d2s", "st": 2, "sh": 1, "sw": 2}],
}


def test_temporal_clip_lines_up_with_the_whole_decode():
    """A temporally local plan pins the frame alignment: each clip decoded alone equals the whole
    decode over the clip's output span, for every clip start."""
    z = np.random.default_rng(3).standard_normal((1, 7, 3, 4, 16))
    whole = oracle.decode(_LOCAL_PLAN, z, [])
    assert whole.shape == (1, 25, 6, 8, 1)
    for s in range(7):
        for n in range(1, 8 - s):
            lo, hi = oracle.tiling.out_span(s, n, 4, True)
            clip = oracle.decode(_LOCAL_PLAN, z[:, s:s + n], [])
            assert np.array_equal(clip, whole[:, lo:hi]), (s, n)


@pytest.mark.parametrize("tt,stt", [(3, 2), (4, 2), (4, 3)])
def test_temporal_overlap_blend_of_a_local_plan_is_the_whole_decode(tt, stt):
    z = np.random.default_rng(4).standard_normal((1, 7, 3, 4, 16))
    whole = oracle.decode(_LOCAL_PLAN, z, [])
    tiled = oracle.decode_overlap_blend(_LOCAL_PLAN, z, [], (2, 3), (1, 2), (4, 2, 2), tt, stt)
    np.testing.assert_allclose(tiled, whole, rtol=1e-14, atol=1e-14)
