"""Pins for the voxel-grid downsampling oracle (CPU only).

The oracle (``oracle.downsample``) is checked against what fixes its result
independently: a numpy grouping implementation on every workload, the
pinned pillar oracle (same voxels, ids and coordinates), closed-form means on
hand-built clouds, and a case where single-precision accumulation gives a
different answer than the double-precision one the definition asks for.
"""
import numpy as np
import pytest

import oracle
from bruteforce import downsample_np, same_f32
from workloads import config_names, generate, get_config

F32 = np.float32
GRID = ((0.0, 0.0, -1.0, 4.0, 4.0, 1.0), (1.0, 1.0, 2.0), (4, 4, 1))


def _check(pts, r, c, g, M):
    got = oracle.downsample(pts, r, c, g, M)
    want = downsample_np(pts, r, c, g, M)
    assert same_f32(got[0], want[0]), "centroids differ"
    assert np.array_equal(got[1], want[1]), "coords differ"
    assert np.array_equal(got[2], want[2]), "counts differ"
    return got


@pytest.mark.parametrize("name", config_names())
def test_downsample_matches_numpy_grouping(name):
    cfg = get_config(name)
    p = cfg.params
    pts, _ = generate(name)
    _check(pts, p.range_, p.cell, p.grid, p.max_voxels)


@pytest.mark.parametrize("name", ["tiny", "kitti_frame", "voxel3d"])
def test_downsample_agrees_with_pillar_oracle(name):
    """Same voxels in the same order as the pinned pillar oracle, and with
    max_points at least the largest voxel, the same counts."""
    cfg = get_config(name)
    p = cfg.params
    pts, _ = generate(name)
    cen, coords, counts = oracle.downsample(pts, p.range_, p.cell, p.grid, p.max_voxels)
    K = int(counts.max()) if counts.size else 1
    _, vc, vn = oracle.voxelize(pts, p.range_, p.cell, p.grid, K, p.max_voxels)
    assert np.array_equal(coords, vc)
    assert np.array_equal(counts, vn)


def test_single_point_voxels_reproduce_the_point():
    """A voxel holding one point has that point as its mean, bit for bit."""
    cfg = get_config("uniform_25k")
    p = cfg.params
    pts, _ = generate("uniform_25k")
    cen, _, counts = oracle.downsample(pts, p.range_, p.cell, p.grid, 10 ** 6)
    vox, _, _ = oracle.voxelize(pts, p.range_, p.cell, p.grid, 1, 10 ** 6)
    one = counts == 1
    assert one.sum() > 1000
    assert np.array_equal(cen[one].view(np.uint32), vox[one, 0].view(np.uint32))


def test_closed_form_means():
    pts = np.array([
        [1.25, 0.5, 0.0, 1.0],    # voxel (1, 0)
        [1.75, 0.25, 0.5, 3.0],   # voxel (1, 0)
        [0.5, 2.5, 0.0, 2.0],     # voxel (0, 2)
        [-0.25, 0.5, 0.0, 9.0],   # rejected (x below the grid)
        [1.5, 0.75, -0.5, 5.0],   # voxel (1, 0)
    ], F32)
    cen, coords, counts = oracle.downsample(pts, *GRID, 8)
    assert coords.tolist() == [[0, 0, 1], [0, 2, 0]]
    assert counts.tolist() == [3, 1]
    assert cen.tolist() == [[1.5, 0.5, 0.0, 3.0], [0.5, 2.5, 0.0, 2.0]]
    # the cap keeps the first voxel by first occurrence only
    cen1, coords1, counts1 = oracle.downsample(pts, *GRID, 1)
    assert coords1.tolist() == [[0, 0, 1]] and counts1.tolist() == [3]
    assert cen1.tolist() == [[1.5, 0.5, 0.0, 3.0]]


def test_double_precision_accumulation_is_what_is_computed():
    """Ten points in one voxel above 1000 whose float32 running sum rounds
    enough to move the mean by one ulp: the definition's double sum does not,
    and the oracle's mean is the double one."""
    x = np.array([1000.269775390625, 1000.0409545898438, 1000.0165405273438,
                  1000.8132934570312, 1000.9127807617188, 1000.6066284179688,
                  1000.7294921875, 1000.5436401367188, 1000.93505859375,
                  1000.8158569335938], F32)
    pts = np.zeros((x.size, 4), F32)
    pts[:, 0] = x
    pts[:, 1] = F32(0.5)
    r, c, g = (999.0, 0.0, -1.0, 1003.0, 4.0, 1.0), (1.0, 1.0, 2.0), (4, 4, 1)
    cen, _, counts = oracle.downsample(pts, r, c, g, 4)
    exact = F32(sum(float(v) for v in x) / x.size)
    s32 = F32(0.0)
    for v in x:
        s32 = F32(s32 + v)
    single = F32(s32 / F32(x.size))
    assert counts.tolist() == [10]
    assert cen[0, 0] == exact == F32(1000.5684204101562)
    assert single != exact  # the case does discriminate


def test_nan_and_inf_intensity_propagate():
    pts = np.array([[0.5, 0.5, 0.0, np.nan], [0.6, 0.5, 0.0, 1.0],
                    [1.5, 0.5, 0.0, np.inf], [1.6, 0.5, 0.0, -np.inf],
                    [2.5, 0.5, 0.0, np.inf]], F32)
    cen, _, counts = oracle.downsample(pts, *GRID, 8)
    assert counts.tolist() == [2, 2, 1]
    assert np.isnan(cen[0, 3]) and np.isnan(cen[1, 3]) and cen[2, 3] == np.inf
    assert _check(pts, *GRID, 8) is not None


def test_empty_and_all_rejected():
    cen, coords, counts = oracle.downsample(np.zeros((0, 4), F32), *GRID, 4)
    assert cen.shape == (0, 4) and coords.shape == (0, 3) and counts.shape == (0,)
    bad = np.array([[np.nan, 0.5, 0, 0], [4.0, 0.5, 0, 0], [0.5, 0.5, 1.0, 0]], F32)
    assert oracle.downsample(bad, *GRID, 4)[0].shape == (0, 4)


def test_integer_valued_points_are_order_free():
    """With small integer-valued coordinates every partial sum is exact, so
    any order of the points gives the same means."""
    rng = np.random.default_rng(3)
    n = 3000
    pts = np.zeros((n, 4), F32)
    pts[:, 0] = rng.integers(0, 64, n).astype(F32)
    pts[:, 1] = rng.integers(0, 64, n).astype(F32)
    pts[:, 3] = rng.integers(-50, 50, n).astype(F32)
    r, c, g = (0.0, 0.0, -1.0, 64.0, 64.0, 1.0), (8.0, 8.0, 2.0), (8, 8, 1)
    a = oracle.downsample(pts, r, c, g, 100)
    perm = rng.permutation(n)
    b = oracle.downsample(pts[perm], r, c, g, 100)
    order_a = np.lexsort(a[1].T[::-1])
    order_b = np.lexsort(b[1].T[::-1])
    assert np.array_equal(a[1][order_a], b[1][order_b])
    assert np.array_equal(a[2][order_a], b[2][order_b])
    assert np.array_equal(a[0][order_a], b[0][order_b])
