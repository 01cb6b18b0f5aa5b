"""The pins must reject a wrong oracle.

Each case copies the oracle's C source, plants one plausible mistake (a
dropped term, a wrong bound, a swapped index, a different rounding), builds it
with the same flags, and runs a battery of the independent pins against it.
The unmodified source must pass the battery and every mutant must fail it.
All of this runs on the CPU.
"""
import json
import os

import numpy as np
import pytest

import oracle
from bruteforce import (bin_np, downsample_np, exact_cell, same_f32, sort_by_voxel_np,
                        sort_then_segment, spherical_np)
from test_oracle_spherical import SMALL, _angles, _boundary_dirs, _rot, _vid
from workloads import generate, get_config, get_sph_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32

MUTANTS = {
    "truncation_instead_of_floor": [("floorf((x - g->x_min) / g->vx)", "truncf((x - g->x_min) / g->vx)")],
    "non_strict_upper_x": [("fx < (float)g->gx", "fx <= (float)g->gx")],
    "non_strict_zslab_top": [("z < z_max", "z <= z_max")],
    "strict_zslab_bottom": [("z >= g->z_min", "z > g->z_min")],
    "non_strict_upper_z_cell": [("fz < (float)g->gz", "fz <= (float)g->gz")],
    "keep_one_point_less": [("total[pid] <= K", "total[pid] < K")],
    "coords_y_gets_x": [("coords[3 * pid + 1] = (int32_t)cy;", "coords[3 * pid + 1] = (int32_t)cx;")],
    "cap_one_short": [("V < max_voxels", "V < max_voxels - 1")],
    "rows_reversed": [("(pid * K + (total[pid] - 1))", "(pid * K + (K - total[pid]))")],
    "key_uses_gx_for_gy": [("(cz * g->gy + cy)", "(cz * g->gx + cy)")],
    "reciprocal_multiply": [("(x - g->x_min) / g->vx", "(x - g->x_min) * (1.0f / g->vx)")],
    "y_divided_by_vx": [("(y - g->y_min) / g->vy", "(y - g->y_min) / g->vx")],
    "no_zero_padding": [("memset(voxels + (pid * K + j) * 4, 0, 4 * sizeof(float));", "(void)0;")],
    "counts_not_clamped": [("num_points[pid] = (int32_t)c;", "num_points[pid] = (int32_t)total[pid];")],
    "double_precision_binning": [("floorf((x - g->x_min) / g->vx)",
                                  "(float)floor(((double)x - (double)g->x_min) / (double)g->vx)")],
    "keep_last_k": [("if (total[pid] <= K) {", "{"),
                    ("(pid * K + (total[pid] - 1))", "(pid * K + (total[pid] - 1) % K)")],
    "x_min_for_y": [("(y - g->y_min) / g->vy", "(y - g->x_min) / g->vy")],
    "map_zero_for_dropped": [("point_pillar[i] = -1;", "point_pillar[i] = 0;")],
    # voxel-grid downsampling
    "ds_float_accumulator": [("sum[4 * pid + c] += (double)p[c];  /* input order, double precision */",
                              "sum[4 * pid + c] = (double)((float)sum[4 * pid + c] + p[c]);")],
    "ds_count_plus_one": [("centroids[4 * pid + c] = (float)(sum[4 * pid + c] / (double)total[pid]);",
                           "centroids[4 * pid + c] = (float)(sum[4 * pid + c] / (double)(total[pid] + 1));")],
    "ds_channel_swap": [("centroids[4 * pid + c] = (float)(sum[4 * pid + c] / (double)total[pid]);",
                         "centroids[4 * pid + c] = (float)(sum[4 * pid + (c ^ 1)] / (double)total[pid]);")],
    "ds_counts_capped_at_1": [("        counts[pid] = (int32_t)total[pid];",
                               "        counts[pid] = 1;")],
    "ds_skip_first_point": [("            continue;  /* its voxel is past the cap */\n        }\n        for (int c = 0; c < 4; c++)",
                             "            continue;  /* its voxel is past the cap */\n        }\n        if (total[pid] == 0 && sum[4 * pid] == 0.0) { total[pid] += 1; continue; }\n        for (int c = 0; c < 4; c++)")],
    # spherical binning and reorder
    "sph_elev_strict": [("(double)b[k].c * z - (double)b[k].s * rxy >= 0.0)",
                         "(double)b[k].c * z - (double)b[k].s * rxy > 0.0)")],
    "sph_azim_strict": [("return dx * py - dy * px >= 0.0;", "return dx * py - dy * px > 0.0;")],
    "sph_elev_args_swapped": [("sph_bin_elev(tb, nt, (double)rxy, (double)z)",
                               "sph_bin_elev(tb, nt, (double)z, (double)rxy)")],
    "sph_r_without_z": [("float r = sqrtf(sxy + zz);", "float r = sqrtf(sxy);")],
    "sph_no_range_class": [("b[k].cls = a < -lim ? -1 : (a > lim ? 1 : 0);", "b[k].cls = 0;")],
    "sph_negative_zero_y": [("    if (y < 0.0)\n        return 0;",
                             "    if (y < 0.0 || (y == 0.0 && signbit(y)))\n        return 0;")],
    "sph_id_axes_swapped": [("((int64_t)fr * nt + it) * np_ + ip", "((int64_t)fr * np_ + ip) * nt + it")],
    "sph_reversed_in_voxel": [("for (int64_t i = 0; i < n; i++) /* counting sort",
                               "for (int64_t i = n - 1; i >= 0; i--) /* counting sort")],
    "sph_origin_azimuth_pi": [("sph_bin_azim(pb, np_, 1.0, 0.0)", "sph_bin_azim(pb, np_, -1.0, 0.0)")],
    "sph_offsets_inclusive": [("        offsets[v] = (int32_t)run;\n        run += cnt[v];\n        cnt[v] = offsets[v];",
                               "        int64_t start = run;\n        run += cnt[v];\n        offsets[v] = (int32_t)run;\n        cnt[v] = start;")],
    "map_only_kept_rows": [("        if (point_pillar)\n            point_pillar[i] = (int32_t)pid;\n        total[pid] += 1;\n        if (total[pid] <= K) {",
                            "        total[pid] += 1;\n        if (total[pid] <= K) {\n            if (point_pillar)\n                point_pillar[i] = (int32_t)pid;")],
}


def _same(a, b):
    va, ca, na = a
    vb, cb, nb = b
    return (va.shape == vb.shape and np.array_equal(ca, cb) and np.array_equal(na, nb)
            and np.array_equal(va.view(np.uint32), vb.view(np.uint32)))


def _battery(lib):
    """Names of the pins that fail for this oracle build."""
    fails = []
    hand = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))
    for key, gkey in (("cases", "grid_4x4"), ("cases_3d", "grid_3d")):
        gs = hand[gkey]
        for case in hand[key]:
            pts = (np.array([[float(v) for v in r] for r in case["points"]], F32)
                   if case["points"] else np.zeros((0, 4), F32))
            vox, coords, counts, pmap = oracle.voxelize_map(pts, gs["range"], gs["cell"],
                                                            gs["grid"], case["max_points"],
                                                            case["max_voxels"], lib=lib)
            ok = (coords.tolist() == case["coords"] and counts.tolist() == case["num_points"]
                  and pmap.tolist() == case["point_pillar"])
            if ok:
                for p, rows in enumerate(case["rows"]):
                    for j, src in enumerate(rows):
                        want = np.zeros(4, F32) if src is None else pts[src]
                        ok &= bool(np.array_equal(vox[p, j].view(np.uint32), want.view(np.uint32)))
            if not ok:
                fails.append("hand:" + case["name"])
    edge = json.load(open(os.path.join(GOLDEN, "edge_points.json")))
    pts, info = generate("tiny")
    gsp = edge["grid"]
    valid, key = oracle.bin_points(pts, gsp["range"], gsp["cell"], gsp["grid"], lib=lib)
    for name, exp in edge["points"].items():
        i = info["edge_index"][name]
        if bool(valid[i]) != exp["kept"]:
            fails.append("edge:" + name)
        elif exp["kept"]:
            cx = exact_cell(pts[i, 0], gsp["range"][0], gsp["cell"][0])
            cy = exact_cell(pts[i, 1], gsp["range"][1], gsp["cell"][1])
            if key[i] != cy * gsp["grid"][0] + cx:
                fails.append("edge_cell:" + name)
    # 3D z boundary
    prm = get_config("voxel3d").params
    z = np.array([np.nextafter(F32(prm.range_[5]), F32(-np.inf))], F32)
    p3 = np.array([[10.0, 1.0, z[0], 0.0]], F32)
    v3, _ = oracle.bin_points(p3, prm.range_, prm.cell, prm.grid, lib=lib)
    if bool(v3[0]) != (exact_cell(z[0], prm.range_[2], prm.cell[2]) < prm.grid[2]):
        fails.append("z3d_boundary")
    # boundary sweep against numpy float32
    for name in ("tiny", "voxel3d"):
        prm = get_config(name).params
        k = np.arange(prm.grid[0] + 1, dtype=np.float64)
        xs = (F32(prm.range_[0]) + k * float(F32(prm.cell[0]))).astype(F32)
        xs = np.concatenate([xs, np.nextafter(xs, F32(np.inf)), np.nextafter(xs, F32(-np.inf))])
        sw = np.zeros((xs.size, 4), F32)
        sw[:, 0] = xs
        sw[:, 1] = F32((prm.range_[1] + prm.range_[4]) / 2)
        sw[:, 2] = F32((prm.range_[2] + prm.range_[5]) / 2)
        ov, ok_ = oracle.bin_points(sw, prm.range_, prm.cell, prm.grid, lib=lib)
        nv, nk = bin_np(sw, prm.range_, prm.cell, prm.grid)
        if not (np.array_equal(ov, nv) and np.array_equal(ok_, nk)):
            fails.append("sweep:" + name)
    # sort-then-segment on workloads and on fixed random tiny grids
    for name, n in (("kitti_frame", None), ("voxel3d", 200000), ("tiny", None)):
        cfg = get_config(name)
        pts, _ = generate(name, n=n)
        p = cfg.params
        got = oracle.voxelize_map(pts, p.range_, p.cell, p.grid, p.max_points, p.max_voxels,
                                  lib=lib)
        want = sort_then_segment(pts, p.range_, p.cell, p.grid, p.max_points, p.max_voxels,
                                 point_map=True)
        if not (_same(got[:3], want[:3]) and np.array_equal(got[3], want[3])):
            fails.append("brute:" + name)
    rng = np.random.default_rng(7)
    for t in range(40):
        gx, gy = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        vx, vy = float(F32(rng.choice([0.16, 0.3, 1.0]))), float(F32(rng.choice([0.1, 0.5, 0.7])))
        n = int(rng.integers(1, 80))
        pts = np.zeros((n, 4), F32)
        pts[:, 0] = ((rng.integers(-1, gx + 1, n) + rng.choice([0.0, 0.5], n)) * vx).astype(F32)
        pts[:, 1] = ((rng.integers(-1, gy + 1, n) + rng.choice([0.0, 0.5], n)) * vy).astype(F32)
        pts[:, 2] = rng.uniform(-3.5, 1.5, n).astype(F32)
        pts[:, 3] = np.arange(n, dtype=F32)
        r = (0.0, 0.0, -3.0, gx * vx, gy * vy, 1.0)
        K, M = int(rng.integers(1, 4)), int(rng.integers(1, 8))
        got = oracle.voxelize(pts, r, (vx, vy, 4.0), (gx, gy, 1), K, M, lib=lib)
        if not _same(got, sort_then_segment(pts, r, (vx, vy, 4.0), (gx, gy, 1), K, M)):
            fails.append("brute:random")
            break
    # voxel-grid downsampling against numpy grouping and a discriminating case
    for name, n in (("kitti_frame", None), ("tiny", None), ("voxel3d", 100000)):
        p = get_config(name).params
        pts, _ = generate(name, n=n)
        got = oracle.downsample(pts, p.range_, p.cell, p.grid, p.max_voxels, lib=lib)
        want = downsample_np(pts, p.range_, p.cell, p.grid, p.max_voxels)
        if not (same_f32(got[0], want[0]) and np.array_equal(got[1], want[1])
                and np.array_equal(got[2], want[2])):
            fails.append("downsample:" + name)
    x = np.array([1000.269775390625, 1000.0409545898438, 1000.0165405273438,
                  1000.8132934570312, 1000.9127807617188, 1000.6066284179688,
                  1000.7294921875, 1000.5436401367188, 1000.93505859375,
                  1000.8158569335938], F32)
    pts = np.zeros((x.size, 4), F32)
    pts[:, 0] = x
    cen, _, _ = oracle.downsample(pts, (999.0, 0.0, -1.0, 1003.0, 4.0, 1.0), (1.0, 1.0, 2.0),
                                  (4, 4, 1), 4, lib=lib)
    if cen.shape != (1, 4) or cen[0, 0] != F32(1000.5684204101562):
        fails.append("downsample:double_sum")
    fails += _sph_battery(lib)
    return fails


def _sph_battery(lib):
    """Spherical binning pins: hand-placed points, boundary directions and a
    float step either side, the atan2 route and a numpy counting sort."""
    fails = []
    pts = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [-1, 0, 0, 0], [0, -1, 0, 0], [1, 1, 1, 0],
                    [0, 0, 1, 0], [0, 0, 0, 0], [2, 0.1, 0, 0], [0, 0, -1, 0],
                    [-1, -0.0, 0, 0], [3.5, -3.5, 0, 0]], F32)
    v, off, order = oracle.spherical(pts, *SMALL, lib=lib)
    want = [_vid(1, 4, 4), _vid(1, 4, 5), _vid(1, 4, 7), _vid(1, 4, 2), _vid(1, 5, 5),
            _vid(1, 7, 4), -1, _vid(2, 4, 4), _vid(1, 0, 4), _vid(1, 4, 7), -1]
    if v.tolist() != want or order.tolist() != [8, 3, 0, 1, 2, 9, 4, 5, 7]:
        fails.append("sph:hand")
    for axis, (lo, hi) in ((2, (-np.pi + 1e-3, np.pi - 1e-3)), (1, (-np.pi / 2 + 1e-3, np.pi / 2 - 1e-3))):
        rows, exp = [], []
        nb = SMALL[2][axis]
        for k, c, s in _boundary_dirs(SMALL[0][axis], SMALL[1][axis], nb, lo, hi):
            for steps, kk in ((0, k), (-1, k - 1), (1, k)):
                cc, ss = _rot(c, s, steps)
                rows.append([2 * cc, 2 * ss, 0.0, 0.0] if axis == 2 else [2 * cc, 0.0, 2 * ss, 0.0])
                ok = 0 <= kk < nb
                exp.append((_vid(0, 4, kk) if axis == 2 else _vid(0, kk, 4)) if ok else -1)
        v, _, _ = oracle.spherical(np.array(rows, F32), *SMALL, lib=lib)
        if _angles(v) != exp:
            fails.append(f"sph:boundary{axis}")
    p = get_sph_config("lidar_scan_64k").params
    pts, _ = generate("lidar_scan_64k")
    v, off, order = oracle.spherical(pts, p.sph_min, p.sph_cell, p.bins, lib=lib)
    vn, amb = spherical_np(pts, p.sph_min, p.sph_cell, p.bins)
    if np.any((v != vn) & ~amb):
        fails.append("sph:atan2")
    offn, ordn = sort_by_voxel_np(v, int(np.prod(p.bins)))
    if not (np.array_equal(off, offn) and np.array_equal(order, ordn)):
        fails.append("sph:sort")
    return fails


def _build(tmp_path, name, edits):
    src = open(oracle.SOURCE).read()
    for old, new in edits:
        assert src.count(old) >= 1, (name, old)
        src = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    out = tmp_path / f"lib{name}.so"
    oracle.build(str(path), str(out))
    return oracle.load(str(out))


def test_unmodified_oracle_passes_battery(tmp_path):
    assert _battery(_build(tmp_path, "control", [])) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    fails = _battery(_build(tmp_path, name, MUTANTS[name]))
    assert fails, f"mutant {name} passes every pin"
