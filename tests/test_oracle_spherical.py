"""Pins for the spherical binning and voxel-contiguous reorder oracle (CPU only).

``oracle.spherical`` follows the preprocessing of the RadiusFPS page
("Spherical voxel partition"; the one-off sort of RadiusFPS-G): spherical
coordinates, uniform splits per axis, points sorted so a voxel's points are
contiguous. Its angle bins use exact direction tests, not a rounded atan2.
These tests pin it to what fixes the result independently:
  - the atan2 route in float64 (``spherical_np``), which must agree on every
    point not within 1e-6 rad of a boundary;
  - hand-placed points on the axes, on boundary directions and one float step
    either side of them (the half-open rule of each bin);
  - a numpy stable counting sort for the offsets and the order.
"""
import math

import numpy as np
import pytest

import oracle
from bruteforce import sort_by_voxel_np, spherical_np
from workloads import generate, get_sph_config, sph_config_names

F32 = np.float32
PI = math.pi
# 4 shells of 1 m, 8 elevation bands of pi/8, 8 azimuth slices of pi/4
SMALL = ((0.0, -PI / 2, -PI), (1.0, PI / 8, PI / 4), (4, 8, 8))


def _vid(ir, it, ip, bins=SMALL[2]):
    return (ir * bins[1] + it) * bins[2] + ip


def _check_against_atan2(pts, sph_min, sph_cell, bins, max_ambiguous):
    v, off, order = oracle.spherical(pts, sph_min, sph_cell, bins)
    vn, amb = spherical_np(pts, sph_min, sph_cell, bins)
    assert not np.any((v != vn) & ~amb), "bins differ away from every boundary"
    assert amb.sum() <= max_ambiguous
    # an ambiguous point may only move to a neighbouring bin along one angle axis
    for i in np.flatnonzero((v != vn) & amb):
        if v[i] < 0 or vn[i] < 0:
            continue
        a, b = int(v[i]), int(vn[i])
        nph = bins[2]
        assert a // (bins[1] * nph) == b // (bins[1] * nph)
        assert abs((a // nph) % bins[1] - (b // nph) % bins[1]) + abs(a % nph - b % nph) == 1
    offn, ordn = sort_by_voxel_np(v, int(np.prod(bins)))
    assert np.array_equal(off, offn)
    assert np.array_equal(order, ordn)
    return v, off, order


@pytest.mark.parametrize("name", sph_config_names())
def test_workloads_match_atan2_route(name):
    cfg = get_sph_config(name)
    p = cfg.params
    pts, _ = generate(name)
    v, off, order = _check_against_atan2(pts, p.sph_min, p.sph_cell, p.bins, pts.shape[0] // 1000)
    assert order.size == off[-1] > 0.8 * pts.shape[0]


def test_random_ball_all_octants():
    """Every direction, a few shells, coarse and fine angle grids."""
    rng = np.random.default_rng(11)
    n = 200000
    d = rng.normal(size=(n, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    pts = np.zeros((n, 4), F32)
    pts[:, :3] = (d * rng.uniform(0.0, 5.0, size=(n, 1))).astype(F32)
    pts[:, 3] = np.arange(n, dtype=F32)
    _check_against_atan2(pts, *SMALL, n // 1000)
    fine = ((0.5, -1.2, -3.0), (0.25, 0.01, 0.013), (16, 240, 461))
    _check_against_atan2(pts, *fine, n // 500)


def test_axis_and_diagonal_points():
    pts = np.array([
        [1, 0, 0, 0],      # r 1, elevation 0, azimuth 0
        [0, 1, 0, 0],      # azimuth pi/2 falls below boundary 6 (float pi/4 steps from float -pi)
        [-1, 0, 0, 0],     # azimuth pi: last slice
        [0, -1, 0, 0],     # azimuth -pi/2
        [1, 1, 1, 0],      # elevation 35.3 deg, azimuth 45 deg, r sqrt(3)
        [0, 0, 1, 0],      # straight up: last band, azimuth 0
        [0, 0, 0, 0],      # origin: no direction
        [2, 0.1, 0, 0],    # r 2.0025
        [0, 0, -1, 0],     # straight down: first band
        [-1, -0.0, 0, 0],  # -0 y counts as +0: azimuth pi
        [3.5, -3.5, 0, 0],  # r 4.95 is past the last shell
    ], F32)
    v, off, order = oracle.spherical(pts, *SMALL)
    want = [_vid(1, 4, 4), _vid(1, 4, 5), _vid(1, 4, 7), _vid(1, 4, 2), _vid(1, 5, 5),
            _vid(1, 7, 4), -1, _vid(2, 4, 4), _vid(1, 0, 4), _vid(1, 4, 7), -1]
    assert v.tolist() == want
    assert order.tolist() == [8, 3, 0, 1, 2, 9, 4, 5, 7]
    assert off[-1] == 9


def test_nonfinite_and_out_of_range_dropped():
    pts = np.array([[np.nan, 1, 0, 0], [1, np.inf, 0, 0], [1, 0, -np.inf, 0],
                    [4.0, 0, 0, 0], [3.9999998, 0, 0, 0], [0.5, 0, 0, np.nan]], F32)
    v, off, order = oracle.spherical(pts, *SMALL)
    assert v.tolist() == [-1, -1, -1, -1, _vid(3, 4, 4), _vid(0, 4, 4)]
    assert order.tolist() == [4, 5] or order.tolist() == [5, 4]
    assert order.tolist() == [5, 4]  # voxel order, then input order


def test_shell_boundaries_half_open():
    """r exactly on a shell boundary goes to the outer shell."""
    pts = np.array([[1.0, 0, 0, 0], [np.nextafter(F32(1.0), F32(0)), 0, 0, 0],
                    [0, 0, 2.0, 0], [0, 0, np.nextafter(F32(2.0), F32(0)), 0]], F32)
    v, _, _ = oracle.spherical(pts, *SMALL)
    assert v.tolist() == [_vid(1, 4, 4), _vid(0, 4, 4), _vid(2, 7, 4), _vid(1, 7, 4)]


def _rot(c, s, steps):
    """Turn direction (c, s) by a few float steps of its smaller component."""
    c, s = F32(c), F32(s)
    for _ in range(abs(steps)):
        if abs(c) >= abs(s):   # move s, which changes the angle fastest
            s = np.nextafter(s, F32(np.inf) if (c > 0) == (steps > 0) else F32(-np.inf))
        else:
            c = np.nextafter(c, F32(-np.inf) if (s > 0) == (steps > 0) else F32(np.inf))
    return float(c), float(s)


def _angles(v):
    """Angle part of each voxel id (the shell of a point at r close to 2 may
    be either side of that shell boundary)."""
    return [int(x) % 64 if x >= 0 else -1 for x in v]


def _boundary_dirs(a_min, da, nb, lo, hi):
    """Float directions of the boundaries strictly inside (lo, hi) (radians)."""
    out = []
    for k in range(nb + 1):
        a = float(F32(a_min)) + k * float(F32(da))
        if lo < a < hi:
            out.append((k, float(F32(math.cos(a))), float(F32(math.sin(a)))))
    return out


def test_points_on_azimuth_boundaries():
    """A point whose direction is a boundary's float direction is in the bin
    above that boundary; turned one float step clockwise it is in the bin
    below. Scaling by 2 keeps the direction exact."""
    a_min, da, nb = SMALL[0][2], SMALL[1][2], SMALL[2][2]
    rows, want = [], []
    for k, c, s in _boundary_dirs(a_min, da, nb, -PI + 1e-3, PI - 1e-3):
        for steps, kk in ((0, k), (-1, k - 1), (1, k)):
            cc, ss = _rot(c, s, steps)
            rows.append([2 * cc, 2 * ss, 0.0, 0.0])
            want.append(_vid(0, 4, kk) if 0 <= kk < nb else -1)
    assert len(rows) >= 3 * (nb - 1)
    v, _, _ = oracle.spherical(np.array(rows, F32), *SMALL)
    assert _angles(v) == want


def test_points_on_elevation_boundaries():
    """Same half-open rule for elevation bands, on the direction
    (sqrt(x*x), z), which equals (x, z) exactly for x > 0."""
    t_min, dt, nt = SMALL[0][1], SMALL[1][1], SMALL[2][1]
    rows, want = [], []
    for k, c, s in _boundary_dirs(t_min, dt, nt, -PI / 2 + 1e-3, PI / 2 - 1e-3):
        for steps, kk in ((0, k), (-1, k - 1), (1, k)):
            cc, ss = _rot(c, s, steps)
            rows.append([2 * cc, 0.0, 2 * ss, 0.0])
            want.append(_vid(0, kk, 4) if 0 <= kk < nt else -1)
    v, _, _ = oracle.spherical(np.array(rows, F32), *SMALL)
    assert _angles(v) == want


def test_azimuth_range_ends():
    """The float parameters put the first boundary below -pi (every azimuth is
    above it) and the last one, -pi + 8 * float(pi/4), above pi (no azimuth
    reaches it), so the slices cover the whole turn; a narrower range drops
    the azimuths past its end."""
    assert float(F32(-PI)) < -PI and float(F32(-PI)) + 8 * float(F32(PI / 4)) > PI
    pts = np.array([[-1, 1e-7, 0, 0], [-1, -1e-7, 0, 0]], F32)
    v, _, _ = oracle.spherical(pts, *SMALL)
    assert v.tolist() == [_vid(1, 4, 7), _vid(1, 4, 0)]
    # azimuth [0, 3 * float(pi/4)): 3 * float(pi/4) is above 3pi/4, so the
    # direction (-1, 1) at exactly 3pi/4 is still in the last slice
    three = ((0.0, -PI / 2, 0.0), (1.0, PI / 8, PI / 4), (4, 8, 3))
    assert 3 * float(F32(PI / 4)) > 3 * PI / 4
    pts = np.array([[1, 1, 0, 0], [1, -1, 0, 0], [-1, 0, 0, 0], [1, 0, 0, 0], [-1, 1, 0, 0]], F32)
    v, _, _ = oracle.spherical(pts, *three)
    base = (1 * 8 + 4) * 3
    assert v.tolist() == [base + 1, -1, -1, base + 0, base + 2]


def test_empty_and_all_dropped():
    v, off, order = oracle.spherical(np.zeros((0, 4), F32), *SMALL)
    assert v.shape == (0,) and order.shape == (0,)
    assert off.shape == (4 * 8 * 8 + 1,) and not off.any()
    v, off, order = oracle.spherical(np.zeros((5, 4), F32), *SMALL)
    assert (v == -1).all() and order.size == 0 and not off.any()


def test_reorder_under_input_permutation():
    """Binning is per point; permuting the input permutes voxel_of and keeps
    the offsets, and the order lists the same points per voxel."""
    cfg = get_sph_config("lidar_scan_64k")
    p = cfg.params
    pts, _ = generate("lidar_scan_64k")
    v, off, order = oracle.spherical(pts, p.sph_min, p.sph_cell, p.bins)
    perm = np.random.default_rng(5).permutation(pts.shape[0])
    v2, off2, order2 = oracle.spherical(pts[perm], p.sph_min, p.sph_cell, p.bins)
    assert np.array_equal(v2, v[perm])
    assert np.array_equal(off2, off)
    for a in np.flatnonzero(np.diff(off) > 0)[:200]:
        seg = order[off[a]:off[a + 1]]
        seg2 = perm[order2[off[a]:off[a + 1]]]
        assert np.array_equal(np.sort(seg), np.sort(seg2))
        assert np.all(np.diff(seg) > 0)
