"""Seeded synthetic point clouds, [N, 4] float32 rows (x, y, z, intensity).

Every cloud is drawn with ``numpy.random.default_rng(seed)`` (PCG64) in a
fixed draw order, so a (config, seed) pair always gives the same bytes. Draws
are i.i.d. per point, so clouds are unordered, like the raw scan the "Voxelize"
page feeds its kernel (Fig. 1 caption). The recipes are the plainest readings
of the workload descriptions; the real KITTI frames the page measures on are
not available, so the KITTI-shaped generator stands in for them.

Nothing here bins, hashes or groups points: the tiny workload's edge points
are placed from the grid's *parameters* (range ends, cell size) with
``nextafter`` where a point must sit one float below a boundary.
"""
from __future__ import annotations

import math
from typing import Dict, List, Tuple

import numpy as np

from .configs import SPH_CONFIGS, Config, get_config, get_sph_config

F32 = np.float32


def _f32_below(v: float) -> float:
    return float(np.nextafter(F32(v), F32(-np.inf)))


def _edge_points() -> List[Tuple[str, Tuple[float, float, float, float]]]:
    """The 32 hand-placed edge points of the tiny workload (pillar grid geometry).

    Each one sits on a boundary or special value that the binning rules of the
    page's "Binning a point" section decide: the NaN/Inf check, the z-slab,
    floor (not truncation) just below the origin, and the strict upper bound.
    Names are stable; the expected outcome of each lives with the tests.
    """
    nan, inf = float("nan"), float("inf")
    x_max, y_min, y_max, z_min, z_max = 69.12, -39.68, 39.68, -3.0, 1.0
    return [
        ("x_eq_xmax", (x_max, 0.0, -1.0, 0.5)),
        ("x_below_xmax", (_f32_below(x_max), 0.0, -1.0, 0.5)),
        ("x_neg_1e-6", (-1e-6, 0.0, -1.0, 0.5)),
        ("x_neg_zero", (-0.0, 0.0, -1.0, 0.5)),
        ("x_neg_denormal", (-1e-40, 0.0, -1.0, 0.5)),
        ("x_nan", (nan, 0.0, -1.0, 0.5)),
        ("y_nan", (10.0, nan, -1.0, 0.5)),
        ("z_nan", (10.0, 0.0, nan, 0.5)),
        ("x_pos_inf", (inf, 0.0, -1.0, 0.5)),
        ("x_neg_inf", (-inf, 0.0, -1.0, 0.5)),
        ("y_pos_inf", (10.0, inf, -1.0, 0.5)),
        ("z_neg_inf", (10.0, 0.0, -inf, 0.5)),
        ("intensity_nan", (20.0, 5.0, -1.0, nan)),
        ("z_eq_zmin", (21.0, 5.0, z_min, 0.5)),
        ("z_eq_zmax", (22.0, 5.0, z_max, 0.5)),
        ("z_below_zmax", (23.0, 5.0, _f32_below(z_max), 0.5)),
        ("x_1e30", (1e30, 0.0, -1.0, 0.5)),
        ("x_neg_1e30", (-1e30, 0.0, -1.0, 0.5)),
        ("y_1e30", (10.0, 1e30, -1.0, 0.5)),
        ("corner_last_cell", (x_max - 0.08, y_max - 0.08, -1.0, 0.5)),
        ("y_eq_ymax", (30.0, y_max, -1.0, 0.5)),
        ("y_eq_ymin", (31.0, y_min, -1.0, 0.5)),
        ("y_below_ymin", (32.0, _f32_below(y_min), -1.0, 0.5)),
        ("z_1e30", (33.0, 5.0, 1e30, 0.5)),
        ("x_pos_denormal", (1e-40, 1.0, -1.0, 0.5)),
        ("intensity_inf", (34.0, 6.0, -1.0, inf)),
        ("intensity_neg_zero", (35.0, 7.0, -1.0, -0.0)),
        ("x_eq_cell", (0.16, 2.0, -1.0, 0.25)),
        ("x_below_cell", (_f32_below(0.16), 2.0, -1.0, 0.75)),
        ("x_eq_cell_duplicate", (0.16, 2.0, -1.0, 0.25)),
        ("x_3e38", (3.0e38, 0.0, -1.0, 0.5)),
        ("last_column_first_row", (69.0, y_min + 0.08, -1.0, 0.5)),
    ]


def edge_point_names() -> List[str]:
    return [n for n, _ in _edge_points()]


def _uniform_box(rng, n, lo, hi):
    return rng.uniform(lo, hi, size=n)


def _tiny(rng, n_uniform: int, cluster: int):
    x = _uniform_box(rng, n_uniform, 0.0, 69.12)
    y = _uniform_box(rng, n_uniform, -39.68, 39.68)
    z = _uniform_box(rng, n_uniform, -3.0, 1.0)
    w = rng.uniform(0.0, 1.0, size=n_uniform)
    base = np.stack([x, y, z, w], axis=1).astype(F32)
    edges = _edge_points()
    edge = np.array([p for _, p in edges], dtype=F32)
    # A cluster of `cluster` points inside one interior cell: the square
    # [32.00, 32.16) x [0.00, 0.16) (cell 200 in x, 248 in y of the pillar grid),
    # jittered by at most 0.04 m around its centre so no point is near an edge.
    cxy = np.array([32.08, 0.08])
    jit = rng.uniform(-0.04, 0.04, size=(cluster, 2))
    cz = rng.uniform(-2.5, 0.5, size=cluster)
    cw = rng.uniform(0.0, 1.0, size=cluster)
    clu = np.column_stack([cxy[0] + jit[:, 0], cxy[1] + jit[:, 1], cz, cw]).astype(F32)
    pts = np.concatenate([base, edge, clu], axis=0)
    perm = rng.permutation(pts.shape[0])
    pts = pts[perm]
    # where each edge point ended up (index into the permuted cloud)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    edge_index = {name: int(inv[n_uniform + k]) for k, (name, _) in enumerate(edges)}
    cluster_index = np.sort(inv[n_uniform + len(edges):]).astype(np.int64)
    return np.ascontiguousarray(pts), dict(edge_index=edge_index, cluster_index=cluster_index)


def _kitti_frame(rng, n: int):
    """KITTI-shaped frame: 90% ground returns ahead of the sensor, 10% clutter."""
    ground = rng.random(n) < 0.9
    phi = rng.uniform(-math.pi / 4, math.pi / 4, size=n)
    # log-uniform range on [2, 80] m: areal density falls as 1/r^2
    r = np.exp(rng.uniform(math.log(2.0), math.log(80.0), size=n))
    zg = np.clip(rng.normal(-1.2, 0.6, size=n), -4.0, 3.0)
    cx = rng.uniform(0.0, 69.12, size=n)
    cy = rng.uniform(-39.68, 39.68, size=n)
    cz = rng.uniform(-4.0, 3.0, size=n)
    w = rng.beta(2.0, 5.0, size=n)
    x = np.where(ground, r * np.cos(phi), cx)
    y = np.where(ground, r * np.sin(phi), cy)
    z = np.where(ground, zg, cz)
    return np.ascontiguousarray(np.stack([x, y, z, w], axis=1).astype(F32))


def _kitti(rng, n: int):
    return _kitti_frame(rng, n), {}


def _uniform(rng, n: int):
    x = _uniform_box(rng, n, 0.0, 69.12)
    y = _uniform_box(rng, n, -39.68, 39.68)
    z = _uniform_box(rng, n, -3.0, 1.0)
    w = rng.uniform(0.0, 1.0, size=n)
    return np.ascontiguousarray(np.stack([x, y, z, w], axis=1).astype(F32)), {}


def _multisweep(rng, frame_n: int, sweeps: int, jitter: float):
    base = _kitti_frame(rng, frame_n).astype(np.float64)
    out = np.empty((frame_n * sweeps, 4), dtype=F32)
    for s in range(sweeps):
        noise = rng.normal(0.0, jitter, size=(frame_n, 3))
        blk = base.copy()
        blk[:, :3] += noise
        out[s * frame_n:(s + 1) * frame_n] = blk.astype(F32)
    return out, {}


def _voxel3d(rng, n: int):
    xs: List[np.ndarray] = []
    ys: List[np.ndarray] = []
    have = 0
    while have < n:
        m = 2 * (n - have) + 1024
        phi = rng.uniform(-math.pi / 2, math.pi / 2, size=m)
        r = np.exp(rng.uniform(math.log(2.0), math.log(80.0), size=m))
        x = r * np.cos(phi)
        y = r * np.sin(phi)
        keep = (x >= 0.0) & (x < 70.4) & (y >= -40.0) & (y < 40.0)
        xs.append(x[keep])
        ys.append(y[keep])
        have += int(keep.sum())
    x = np.concatenate(xs)[:n]
    y = np.concatenate(ys)[:n]
    z = rng.uniform(-3.0, 1.0, size=n)
    w = rng.uniform(0.0, 1.0, size=n)
    return np.ascontiguousarray(np.stack([x, y, z, w], axis=1).astype(F32)), {}


def _lidar_scan(rng, n: int):
    """A 64-beam spinning LiDAR at the origin, 1.73 m above flat ground.

    Beam elevations are spread evenly over [-24.9, 2.0] degrees (jittered by
    0.02 degrees), azimuth is uniform over the full turn. A beam returns from
    the ground where it points down and meets it, or from an obstacle at a
    log-uniform range in [1, 120] m (drawn for 40% of the rays) when that is
    nearer; rays with neither return at 120 m. Range noise is 2 cm.
    """
    beam = rng.integers(0, 64, size=n)
    elev = np.radians(-24.9 + 26.9 * beam / 63.0 + rng.normal(0.0, 0.02, size=n))
    az = rng.uniform(-math.pi, math.pi, size=n)
    down = np.maximum(-np.sin(elev), 1e-9)
    ground = np.where(elev < 0.0, 1.73 / down, np.inf)
    obstacle = np.where(rng.random(n) < 0.4,
                        np.exp(rng.uniform(math.log(1.0), math.log(120.0), size=n)), np.inf)
    r = np.minimum(np.minimum(ground, obstacle), 120.0) + rng.normal(0.0, 0.02, size=n)
    x = r * np.cos(elev) * np.cos(az)
    y = r * np.cos(elev) * np.sin(az)
    z = r * np.sin(elev)
    w = rng.beta(2.0, 5.0, size=n)
    return np.ascontiguousarray(np.stack([x, y, z, w], axis=1).astype(F32)), {}


_GENERATORS = dict(tiny=_tiny, kitti=_kitti, uniform=_uniform, multisweep=_multisweep,
                   voxel3d=_voxel3d, lidar_scan=_lidar_scan)


def generate(config, seed: int | None = None, n: int | None = None) -> Tuple[np.ndarray, Dict]:
    """Return ``(points [N,4] float32, info)`` for a workload name or Config.

    ``seed`` overrides the workload's seed. ``n`` overrides the point count of
    the generators that take one (kitti, uniform, voxel3d) so tests can draw a
    smaller cloud with the same shape. ``info`` carries the tiny workload's
    edge-point positions; it is empty otherwise.
    """
    if isinstance(config, str):
        cfg = get_sph_config(config) if config in SPH_CONFIGS else get_config(config)
    else:
        cfg = config
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    kw = dict(cfg.gen_kwargs)
    if n is not None:
        if "n" not in kw:
            raise ValueError(f"generator {cfg.generator!r} has no point-count override")
        kw["n"] = int(n)
    pts, info = _GENERATORS[cfg.generator](rng, **kw)
    assert pts.dtype == F32 and pts.ndim == 2 and pts.shape[1] == 4 and pts.flags.c_contiguous
    return pts, info
