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
