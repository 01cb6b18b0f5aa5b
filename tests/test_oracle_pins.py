"""Pins for the CPU oracle: each checks it against something other than itself.

* golden edge points: the binning rules of the "Voxelize" page ("Binning a
  point"), with cell indices re-derived by exact rational IEEE arithmetic;
* golden hand-built clouds: expected tensors derived by hand from the page's
  rules (ordering, truncation, the cap, floor vs truncation, 3D mode);
* an independent numpy float32 binning, on boundary sweeps (k*v +- ulps);
* the page's naive method (sort every point by cell id, then segment),
  bit for bit on all five workloads and on fuzzed tiny grids;
* numpy's ``unique`` (no cap, no truncation);
* a closed form for the number of occupied cells of a uniform cloud;
* invariants that hold for any input.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from bruteforce import bin_np, decode, exact_cell, sort_then_segment
from workloads import generate, get_config, config_names

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _as_points(rows):
    if not rows:
        return np.zeros((0, 4), F32)
    return np.array([[float(v) for v in r] for r in rows], dtype=F32)


def assert_same(a, b):
    """Bitwise equality of (voxels, coords, counts) triples."""
    va, ca, na = a
    vb, cb, nb = b
    assert va.shape == vb.shape, (va.shape, vb.shape)
    assert np.array_equal(ca, cb)
    assert np.array_equal(na, nb)
    assert np.array_equal(va.view(np.uint32), vb.view(np.uint32))


# ---------------------------------------------------------------- golden -----

def test_edge_points_follow_page_rules():
    g = _load("edge_points.json")
    cfg = get_config("tiny")
    pts, info = generate("tiny")
    rng, cell, grid = g["grid"]["range"], g["grid"]["cell"], g["grid"]["grid"]
    assert tuple(rng) == cfg.params.range_ and tuple(grid) == cfg.params.grid
    valid, key = oracle.bin_points(pts, rng, cell, grid)
    for name, exp in g["points"].items():
        i = info["edge_index"][name]
        assert bool(valid[i]) == exp["kept"], (name, exp["rule"])
        if exp["kept"]:
            cx = exact_cell(pts[i, 0], rng[0], cell[0])
            cy = exact_cell(pts[i, 1], rng[1], cell[1])
            assert key[i] == cy * grid[0] + cx, name


def test_edge_points_in_tiny_output():
    """Kept edge points appear in the pillar of their cell; rejected ones nowhere."""
    g = _load("edge_points.json")
    cfg = get_config("tiny")
    pts, info = generate("tiny")
    vox, coords, counts = oracle.voxelize_params(pts, cfg.params)
    by_cell = {(int(c[1]), int(c[2])): p for p, c in enumerate(coords)}
    rows_u32 = vox.view(np.uint32)
    for name, exp in g["points"].items():
        i = info["edge_index"][name]
        bits = pts[i].view(np.uint32)
        if exp["kept"]:
            cx = exact_cell(pts[i, 0], 0.0, 0.16)
            cy = exact_cell(pts[i, 1], -39.68, 0.16)
            p = by_cell[(cy, cx)]
            assert any(np.array_equal(rows_u32[p, j], bits) for j in range(counts[p])), name
        else:
            hits = np.all(rows_u32[:, :, :] == bits[None, None, :], axis=2)
            valid_rows = np.arange(cfg.params.max_points)[None, :] < counts[:, None]
            assert not np.any(hits & valid_rows), name


def test_tiny_cluster_truncated_to_lowest_indices():
    cfg = get_config("tiny")
    pts, info = generate("tiny")
    vox, coords, counts = oracle.voxelize_params(pts, cfg.params)
    clu = info["cluster_index"]
    assert clu.size == 40
    p = [k for k, c in enumerate(coords) if (c[1], c[2]) == (248, 200)]
    assert len(p) == 1
    p = p[0]
    assert counts[p] == 32
    want = pts[clu[:32]]
    assert np.array_equal(vox[p].view(np.uint32), want.view(np.uint32))


def _run_hand_case(case, grid_spec):
    pts = _as_points(case["points"])
    out = oracle.voxelize_map(pts, grid_spec["range"], grid_spec["cell"], grid_spec["grid"],
                              case["max_points"], case["max_voxels"])
    vox, coords, counts, pmap = out
    assert pmap.tolist() == case["point_pillar"], case["name"]
    K = case["max_points"]
    V = len(case["coords"])
    assert vox.shape == (V, K, 4), case["name"]
    assert coords.tolist() == case["coords"], case["name"]
    assert counts.tolist() == case["num_points"], case["name"]
    for p, rows in enumerate(case["rows"]):
        for j, src in enumerate(rows):
            want = np.zeros(4, F32) if src is None else pts[src]
            assert np.array_equal(vox[p, j].view(np.uint32), want.view(np.uint32)), \
                (case["name"], p, j)


@pytest.mark.parametrize("case", _load("hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    _run_hand_case(case, _load("hand_cases.json")["grid_4x4"])


@pytest.mark.parametrize("case", _load("hand_cases.json")["cases_3d"], ids=lambda c: c["name"])
def test_hand_cases_3d(case):
    _run_hand_case(case, _load("hand_cases.json")["grid_3d"])


# ---------------------------------------------------- independent binning ----

def _boundary_sweep(lo, v, g, other):
    """Points at k*v + lo and 1-2 floats either side, for every k in [0, g]."""
    k = np.arange(0, g + 1, dtype=np.float64)
    base = (F32(lo) + (k * float(F32(v)))).astype(F32)
    vals = [base]
    up, dn = base, base
    for _ in range(2):
        up = np.nextafter(up, F32(np.inf))
        dn = np.nextafter(dn, F32(-np.inf))
        vals += [up, dn]
    vals = np.concatenate(vals).astype(F32)
    return vals, np.full(vals.shape, other, dtype=F32)


@pytest.mark.parametrize("name", ["tiny", "dense_multisweep", "voxel3d"])
def test_boundary_sweep_matches_numpy_float32(name):
    prm = get_config(name).params
    r, c, g = prm.range_, prm.cell, prm.grid
    xs, ys = _boundary_sweep(r[0], c[0], g[0], F32((r[1] + r[4]) / 2))
    ys2, xs2 = _boundary_sweep(r[1], c[1], g[1], F32((r[0] + r[3]) / 2))
    zs3, _ = _boundary_sweep(r[2], c[2], max(g[2], 1), F32(0))
    n1, n2, n3 = xs.size, ys2.size, zs3.size
    pts = np.zeros((n1 + n2 + n3, 4), F32)
    pts[:n1, 0], pts[:n1, 1], pts[:n1, 2] = xs, ys, F32((r[2] + r[5]) / 2)
    pts[n1:n1 + n2, 0], pts[n1:n1 + n2, 1], pts[n1:n1 + n2, 2] = xs2, ys2, F32((r[2] + r[5]) / 2)
    pts[n1 + n2:, 0], pts[n1 + n2:, 1], pts[n1 + n2:, 2] = F32(r[3] / 2), F32(0), zs3
    ov, ok_ = oracle.bin_points(pts, r, c, g)
    nv, nk = bin_np(pts, r, c, g)
    assert np.array_equal(ov, nv)
    assert np.array_equal(ok_, nk)
    # both sides of every boundary are exercised
    assert ov.sum() > 0 and (~ov).sum() > 0


@pytest.mark.parametrize("name", config_names())
def test_binning_matches_numpy_float32_on_workloads(name):
    cfg = get_config(name)
    pts, _ = generate(name)
    ov, ok_ = oracle.bin_points(pts, cfg.params.range_, cfg.params.cell, cfg.params.grid)
    nv, nk = bin_np(pts, cfg.params.range_, cfg.params.cell, cfg.params.grid)
    assert np.array_equal(ov, nv)
    assert np.array_equal(ok_, nk)


def test_3d_z_boundaries_exact():
    """In 3D mode a point one float below z_max can still floor into cell gz."""
    prm = get_config("voxel3d").params
    r, c, g = prm.range_, prm.cell, prm.grid
    zs = np.array([r[2], np.nextafter(F32(r[5]), F32(-np.inf)), r[5],
                   np.nextafter(F32(r[2]), F32(np.inf)), -2.95, 0.55], dtype=F32)
    pts = np.zeros((zs.size, 4), F32)
    pts[:, 0], pts[:, 1], pts[:, 2] = F32(10.0), F32(1.0), zs
    valid, key = oracle.bin_points(pts, r, c, g)
    for i, z in enumerate(zs):
        in_slab = F32(r[2]) <= z < F32(r[5])
        cz = exact_cell(z, r[2], c[2])
        want = in_slab and 0 <= cz < g[2]
        assert bool(valid[i]) == want, (float(z), cz)
        if want:
            cx = exact_cell(pts[i, 0], r[0], c[0])
            cy = exact_cell(pts[i, 1], r[1], c[1])
            assert key[i] == (cz * g[1] + cy) * g[0] + cx


# ------------------------------------------------- sort then segment ---------

@pytest.mark.parametrize("name", config_names())
def test_oracle_matches_sort_then_segment(name):
    cfg = get_config(name)
    pts, _ = generate(name)
    p = cfg.params
    got = oracle.voxelize_map(pts, p.range_, p.cell, p.grid, p.max_points, p.max_voxels)
    want = sort_then_segment(pts, p.range_, p.cell, p.grid, p.max_points, p.max_voxels,
                             point_map=True)
    assert_same(got[:3], want[:3])
    assert np.array_equal(got[3], want[3])
    # the map agrees with the tensors: every listed row belongs to its pillar
    assert got[3].max() < got[1].shape[0] and (got[3] >= -1).all()


@st.composite
def tiny_problem(draw):
    gx = draw(st.integers(1, 8))
    gy = draw(st.integers(1, 8))
    gz = draw(st.sampled_from([1, 1, 2, 3]))
    vx = float(F32(draw(st.sampled_from([0.1, 0.16, 0.25, 0.3, 1.0, 0.7]))))
    vy = float(F32(draw(st.sampled_from([0.1, 0.16, 0.2, 0.5, 1.0, 0.33]))))
    vz = float(F32(draw(st.sampled_from([0.1, 0.4, 1.0]))))
    x0 = float(F32(draw(st.sampled_from([0.0, -1.0, -0.37, 2.5]))))
    y0 = float(F32(draw(st.sampled_from([0.0, -39.68, 1.1]))))
    z0 = float(F32(draw(st.sampled_from([-3.0, 0.0]))))
    z1 = z0 + (gz * vz if gz > 1 else 4.0)
    n = draw(st.integers(0, 120))
    seed = draw(st.integers(0, 2**31 - 1))
    K = draw(st.integers(1, 4))
    M = draw(st.integers(1, 10))
    rng = np.random.default_rng(seed)
    # points concentrated on a handful of cells plus exact boundaries
    fx = rng.integers(-1, gx + 2, size=n) + rng.choice([0.0, 0.5, 0.999, 1e-7], size=n)
    fy = rng.integers(-1, gy + 2, size=n) + rng.choice([0.0, 0.5, 0.999], size=n)
    fz = rng.uniform(-0.2, 1.2, size=n)
    pts = np.zeros((n, 4), F32)
    pts[:, 0] = (x0 + fx * vx).astype(F32)
    pts[:, 1] = (y0 + fy * vy).astype(F32)
    pts[:, 2] = (z0 + fz * (z1 - z0)).astype(F32)
    pts[:, 3] = np.arange(n, dtype=F32)
    if n:
        bad = rng.random(n) < 0.05
        pts[bad, rng.integers(0, 3)] = np.nan
    rng_ = (x0, y0, z0, x0 + gx * vx, y0 + gy * vy, z1)
    return pts, rng_, (vx, vy, vz), (gx, gy, gz), K, M


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_problem())
def test_oracle_matches_sort_then_segment_fuzzed(prob):
    pts, r, c, g, K, M = prob
    got = oracle.voxelize_map(pts, r, c, g, K, M)
    want = sort_then_segment(pts, r, c, g, K, M, point_map=True)
    assert_same(got[:3], want[:3])
    assert np.array_equal(got[3], want[3])


# ---------------------------------------------------------- np.unique --------

@pytest.mark.parametrize("name", ["tiny", "kitti_frame", "uniform_130k"])
def test_np_unique_without_cap_or_truncation(name):
    cfg = get_config(name)
    pts, _ = generate(name)
    p = cfg.params
    valid, key = bin_np(pts, p.range_, p.cell, p.grid)
    idx = np.flatnonzero(valid)
    uniq, first, cnt = np.unique(key[idx], return_index=True, return_counts=True)
    order = np.argsort(idx[first])
    K = int(cnt.max())
    M = int(uniq.size)
    vox, coords, counts = oracle.voxelize(pts, p.range_, p.cell, p.grid, K, M)
    assert np.array_equal(coords, decode(uniq[order], p.grid))
    assert np.array_equal(counts, cnt[order])


# ---------------------------------------------------------- closed form ------

@pytest.mark.parametrize("name", ["uniform_25k", "uniform_65536", "uniform_130k"])
def test_uniform_occupancy_closed_form(name):
    """E[occupied] = G (1 - (1 - 1/G)^N) for N uniform points over G cells."""
    cfg = get_config(name)
    pts, _ = generate(name)
    p = cfg.params
    G = p.grid[0] * p.grid[1]
    N = pts.shape[0]
    expect = G * (1.0 - (1.0 - 1.0 / G) ** N)
    # variance of the number of occupied cells (occupancy problem)
    q1 = (1.0 - 1.0 / G) ** N
    q2 = (1.0 - 2.0 / G) ** N
    var = G * q1 + G * (G - 1) * q2 - (G * q1) ** 2
    _, coords, _ = oracle.voxelize(pts, p.range_, p.cell, p.grid, 1, G)
    assert abs(coords.shape[0] - expect) < 6 * math.sqrt(var) + 1


# ---------------------------------------------------------- invariants -------

@pytest.mark.parametrize("name", config_names())
def test_invariants(name):
    cfg = get_config(name)
    pts, _ = generate(name)
    p = cfg.params
    tagged = pts.copy()
    tagged[:, 3] = np.arange(pts.shape[0], dtype=F32)   # intensity = index (exact < 2^24)
    vox, coords, counts = oracle.voxelize_params(tagged, p)
    V, K = vox.shape[0], p.max_points
    valid, key = bin_np(tagged, p.range_, p.cell, p.grid)
    # coordinates are unique and inside the grid
    flat = (coords[:, 0].astype(np.int64) * p.grid[1] + coords[:, 1]) * p.grid[0] + coords[:, 2]
    assert np.unique(flat).size == V
    assert (coords[:, 2] < p.grid[0]).all() and (coords[:, 1] < p.grid[1]).all()
    assert (coords[:, 0] < p.grid[2]).all() and (coords >= 0).all()
    # every row bins to its pillar; indices increase; padding is zero
    j = np.arange(K)[None, :]
    live = j < counts[:, None]
    idx = vox[:, :, 3].astype(np.int64)
    assert np.array_equal(key[idx[live]], np.repeat(flat, counts))
    d = np.diff(np.where(live, idx, np.iinfo(np.int64).max), axis=1)
    assert (d[live[:, 1:]] > 0).all()
    assert not vox.view(np.uint32)[~live].any()
    # first indices increase with the pillar id
    assert (np.diff(idx[:, 0]) > 0).all()
    # counts = min(total, K); the V pillars are the first V distinct cells
    uniq, first, cnt = np.unique(key[valid], return_index=True, return_counts=True)
    firsts = np.flatnonzero(valid)[first]
    order = np.argsort(firsts)
    assert V == min(uniq.size, p.max_voxels)
    assert np.array_equal(flat, uniq[order][:V])
    assert np.array_equal(counts, np.minimum(cnt[order][:V], K))
