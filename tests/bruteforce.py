"""Independent checks for the oracle (test-only; shares no code with it).

``bin_np`` evaluates the binning rules of the "Voxelize" page ("Binning a
point") with vectorised numpy float32 operations; ``sort_then_segment`` groups
points the way the page's "Design Decisions" section describes the naive
method: sort every point by its cell id, then cut the sorted list into
segments. Segments are then ordered by their lowest point index, the first
``max_voxels`` are kept and each keeps its ``max_points`` lowest indices.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32 = np.float32


def bin_np(points, range_, cell, grid):
    p = np.asarray(points, dtype=F32)
    x, y, z = p[:, 0], p[:, 1], p[:, 2]
    x0, y0, z0, _, _, z1 = (F32(v) for v in range_)
    vx, vy, vz = (F32(v) for v in cell)
    gx, gy, gz = (int(v) for v in grid)
    with np.errstate(all="ignore"):
        ok = np.isfinite(x) & np.isfinite(y) & np.isfinite(z)
        ok &= (z >= z0) & (z < z1)
        fx = np.floor((x - x0) / vx)
        fy = np.floor((y - y0) / vy)
        ok &= (fx >= F32(0)) & (fx < F32(gx)) & (fy >= F32(0)) & (fy < F32(gy))
        if gz > 1:
            fz = np.floor((z - z0) / vz)
            ok &= (fz >= F32(0)) & (fz < F32(gz))
        else:
            fz = np.zeros_like(fx)
    cx = np.where(ok, fx, 0).astype(np.int64)
    cy = np.where(ok, fy, 0).astype(np.int64)
    cz = np.where(ok, fz, 0).astype(np.int64)
    key = np.where(ok, (cz * gy + cy) * gx + cx, -1)
    return ok, key


def decode(key, grid):
    gx, gy, _ = (int(v) for v in grid)
    key = np.asarray(key, dtype=np.int64)
    cx = key % gx
    cy = (key // gx) % gy
    cz = key // (gx * gy)
    return np.stack([cz, cy, cx], axis=1).astype(np.int32)


def sort_then_segment(points, range_, cell, grid, max_points, max_voxels, point_map=False):
    """Brute-force voxelization: (voxels [V,K,4], coords [V,3], counts [V]), and
    with point_map=True also the per-point pillar id of kept pillars (else -1)."""
    p = np.ascontiguousarray(points, dtype=F32)
    K, M = int(max_points), int(max_voxels)
    ok, key = bin_np(p, range_, cell, grid)
    idx = np.flatnonzero(ok)
    k = key[idx]
    order = np.argsort(k, kind="stable")          # sort by cell id; ties keep index order
    ks, js = k[order], idx[order]
    n = ks.size
    if n == 0:
        out = (np.zeros((0, K, 4), F32), np.zeros((0, 3), np.int32), np.zeros((0,), np.int32))
        return out + (np.full(p.shape[0], -1, np.int32),) if point_map else out
    start_flag = np.r_[True, ks[1:] != ks[:-1]]
    starts = np.flatnonzero(start_flag)
    seg_of = np.cumsum(start_flag) - 1
    seg_len = np.diff(np.r_[starts, n])
    seg_first = js[starts]                         # lowest index of each segment
    seg_rank = np.empty(starts.size, dtype=np.int64)
    seg_rank[np.argsort(seg_first, kind="stable")] = np.arange(starts.size)
    V = min(starts.size, M)
    pos = np.arange(n) - starts[seg_of]
    rank = seg_rank[seg_of]
    take = (rank < V) & (pos < K)
    voxels = np.zeros((V, K, 4), dtype=F32)
    voxels.view(np.uint32)[rank[take], pos[take]] = p.view(np.uint32)[js[take]]
    kept_seg = np.flatnonzero(seg_rank < V)
    coords = np.zeros((V, 3), np.int32)
    counts = np.zeros((V,), np.int32)
    coords[seg_rank[kept_seg]] = decode(ks[starts[kept_seg]], grid)
    counts[seg_rank[kept_seg]] = np.minimum(seg_len[kept_seg], K)
    if point_map:
        pmap = np.full(p.shape[0], -1, np.int32)
        pmap[js] = np.where(rank < V, rank, -1)
        return voxels, coords, counts, pmap
    return voxels, coords, counts


# ---- exact IEEE float32 evaluation with rationals (boundary points) --------

def round_f32(q: Fraction) -> F32:
    """Round a rational to the nearest float32, ties to even (exactly)."""
    c = F32(float(q))
    best = None
    for cand in (np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        if best is None or d < best[0] or (d == best[0] and (int(cand.view(np.uint32)) & 1) == 0):
            best = (d, cand)
    return F32(best[1])


def exact_cell(v, v0, cell) -> int:
    """floor(fl32(fl32(v - v0) / cell)) evaluated with exact rationals."""
    diff = round_f32(Fraction(float(F32(v))) - Fraction(float(F32(v0))))
    quo = round_f32(Fraction(float(diff)) / Fraction(float(F32(cell))))
    return int(np.floor(float(quo)))


# ---- voxel-grid downsampling by grouping (numpy) ---------------------------

def downsample_np(points, range_, cell, grid, max_voxels):
    """Per-voxel means by numpy grouping: binning by ``bin_np``, voxels
    numbered by first occurrence (``np.unique``) and capped at max_voxels,
    x/y/z/intensity summed in float64 with ``np.add.at`` (unbuffered, one
    index after the other, i.e. in input order), divided by the counts in
    float64 and rounded once to float32."""
    p = np.ascontiguousarray(points, dtype=F32)
    valid, key = bin_np(p, range_, cell, grid)
    idx = np.flatnonzero(valid)
    if idx.size == 0:
        return np.zeros((0, 4), F32), np.zeros((0, 3), np.int32), np.zeros((0,), np.int32)
    k = key[idx]
    uk, first, inv = np.unique(k, return_index=True, return_inverse=True)
    order = np.argsort(first, kind="stable")        # voxels by first occurrence
    rank = np.empty_like(order)
    rank[order] = np.arange(order.size)
    pid = rank[inv.reshape(-1)]
    V = min(uk.size, int(max_voxels))
    keep = pid < V
    sums = np.zeros((V, 4), np.float64)
    with np.errstate(invalid="ignore"):  # inf + -inf intensity sums are NaN
        np.add.at(sums, pid[keep], p[idx[keep]].astype(np.float64))
    counts = np.bincount(pid[keep], minlength=V)
    with np.errstate(invalid="ignore"):
        cen = (sums / counts[:, None].astype(np.float64)).astype(F32)
    coords = decode(uk[order[:V]], grid)
    return cen, coords, counts.astype(np.int32)


def same_f32(a, b) -> bool:
    """Bitwise equality of float32 arrays, except that any NaN equals any NaN."""
    a = np.asarray(a, F32)
    b = np.asarray(b, F32)
    if a.shape != b.shape:
        return False
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and
                np.array_equal(a.view(np.uint32)[~na], b.view(np.uint32)[~nb]))


# ----------------------------------------------------------- spherical binning --

def spherical_np(points, sph_min, sph_cell, bins, eps=1e-6):
    """Spherical bins by the atan2 route, in float64, from the float32 direction.

    r is binned with the float32 rules of "Binning a point" on
    r = sqrt((x*x + y*y) + z*z). Elevation is atan2(z, sqrt(x*x + y*y)) and
    azimuth atan2(y, x) (a -0 y taken as +0, azimuth 0 at x = y = 0), both in
    float64 on the float32 values, binned by floor((a - a_min) / da) with
    a_min and da the float32 parameters widened to float64. This route never
    forms a boundary direction, so near a boundary it can disagree with an
    exact direction test: ``ambiguous`` marks points whose angle lies within
    ``eps`` radians of one, where either neighbouring bin is acceptable.
    Returns (voxel id or -1, ambiguous).
    """
    p = np.asarray(points, dtype=F32)
    x, y, z = p[:, 0], p[:, 1], p[:, 2]
    nr, nt, nph = (int(v) for v in bins)
    r0, t0, p0 = (float(F32(v)) for v in sph_min)
    dr32 = F32(sph_cell[0])
    dt, dp = float(F32(sph_cell[1])), float(F32(sph_cell[2]))
    with np.errstate(all="ignore"):
        ok = np.isfinite(x) & np.isfinite(y) & np.isfinite(z)
        sxy = x * x + y * y
        r = np.sqrt(sxy + z * z)
        rxy = np.sqrt(sxy)
        ok &= r != F32(0)
        fr = np.floor((r - F32(r0)) / dr32)
        ok &= (fr >= F32(0)) & (fr < F32(nr))
        th = np.arctan2(z.astype(np.float64), rxy.astype(np.float64))
        yy = y.astype(np.float64) + 0.0
        ph = np.where((x == 0) & (y == 0), 0.0, np.arctan2(yy, x.astype(np.float64)))
        it = np.floor((th - t0) / dt)
        ip = np.floor((ph - p0) / dp)
        ok &= (it >= 0) & (it < nt) & (ip >= 0) & (ip < nph)
        amb = np.zeros(p.shape[0], dtype=bool)
        for a, a0, da, nb in ((th, t0, dt, nt), (ph, p0, dp, nph)):
            kb = np.round((a - a0) / da)
            near = np.abs(a - (a0 + kb * da)) < eps
            amb |= np.isfinite(a) & near & (kb >= 0) & (kb <= nb)
    v = np.where(ok, (fr.astype(np.int64) * nt + np.where(ok, it, 0).astype(np.int64)) * nph
                 + np.where(ok, ip, 0).astype(np.int64), -1)
    return v.astype(np.int64), amb & np.isfinite(r) & (r != F32(0))


def sort_by_voxel_np(voxel_of, nvox):
    """Counting sort by voxel id with numpy: (offsets [nvox+1], order [n_kept]),
    points of one voxel in input order."""
    v = np.asarray(voxel_of, dtype=np.int64)
    kept = np.flatnonzero(v >= 0)
    counts = np.bincount(v[kept], minlength=nvox)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = kept[np.argsort(v[kept], kind="stable")]
    return offsets, order
