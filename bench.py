"""Benchmark: pillar voxelization throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

A step is one complete voxelize call (claim, partition, bins on the default
route; insert, rank, select, pack on the others) over one synthetic cloud
already resident in HBM, outputs and workspace pre-allocated. W untimed
steps, then K steps timed with HIP events on the call's stream, bracketed by
device synchronisation (the page's protocol: mean over timed iterations
after warm-up, inputs on the GPU). Prints one JSON line on stdout.

* value: Mpoints/s = N / (mean time per call), N counting every input point.
* timing: mean, median, p10 and p90 of per-call HIP event times, and the
  wall time per call including the read-back of V to the host.
* roofline: the dominant kernel (largest mean stage time, measured live with
  HIP events around each kernel) against MI355X's 8 TB/s HBM peak, using the
  kernel's algorithmic bytes per launch; `bound` says what limits it.
* cpu_baseline: the C oracle (one thread) on the same cloud on this host,
  with the NumPy sort-then-segment brute force timed beside it, the CPU
  model and the process affinity.
* By default one extra JSON line per voxelization workload goes to stderr
  (every config of the benchmark set); --all adds downsampling and the
  spherical reorder, --spherical only the latter.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "kitti_frame"
METRIC = "Mpoints/s voxelized + achieved HBM GB/s (fraction of peak) at 122,880-pt frame"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--all", action="store_true",
                    help="also time downsampling and the spherical reorder (stderr)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload voxelization lines (stderr)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bound on the oracle's CPU sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline leg")
    ap.add_argument("--downsample", action="store_true",
                    help="also time voxel-grid downsampling of --workload (stderr line)")
    ap.add_argument("--spherical", action="store_true",
                    help="also time the spherical binning and reorder per workload (stderr)")
    ap.add_argument("--profile-iters", type=int, default=50)
    ap.add_argument("--options", default="{}",
                    help="voxelize options as JSON, e.g. '{\"lane_merge\": 1}' (A/B under a profiler)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run 10 plain device copies of this many MiB (counter calibration)")
    ap.add_argument("--rocprof-summary", metavar="DIR", default=None,
                    help="only summarise rocprofv3 CSV output found under DIR (no GPU)")
    return ap.parse_args()


def copy_probe(mib):
    """Plain device-to-device copies of a known size: what FETCH_SIZE and
    WRITE_SIZE read for them calibrates the counters (bytes per counted KiB)."""
    import torch
    n = (mib << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "copies": 10}), flush=True)


def rocprof_summary(root):
    """Per-kernel mean duration (kernel-trace stats) and, when present, mean
    per-dispatch counter values, for the library's kernels and plain copies."""
    import csv
    import glob
    import re
    out = []
    for f in sorted(glob.glob(os.path.join(root, "**", "*kernel_stats.csv"), recursive=True)):
        out.append(f"# {os.path.relpath(f, root)}")
        out.append(f"{'kernel':28s} {'calls':>7s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s}")
        for r in csv.DictReader(open(f)):
            m = re.search(r"k_(\w+)(<[^>]*>)?\(", r["Name"])
            name = "k_" + m.group(1) + (m.group(2) or "") if m else r["Name"][:28]
            out.append(f"{name:28s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.2f} "
                       f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
    for f in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        acc = {}
        for r in csv.DictReader(open(f)):
            m = re.search(r"k_(\w+)(<[^>]*>)?\(", r["Kernel_Name"])
            if m:
                name = "k_" + m.group(1) + (m.group(2) or "")
            elif "copy" in r["Kernel_Name"].lower():
                name = "copy(" + r["Grid_Size"] + ")"
            else:
                continue
            key = (name, r["Counter_Name"])
            d = acc.setdefault(key, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if acc:
            out.append(f"# {os.path.relpath(f, root)} (mean per dispatch, summed over instances)")
            for (name, cn), d in sorted(acc.items()):
                vals = list(d.values())
                out.append(f"{name:28s} {cn:24s} {sum(vals) / len(vals):14.1f}  (dispatches {len(vals)})")
    print("\n".join(out))


def algorithmic_bytes(N, P, V, K, rows, kept, staged, route):
    """Compulsory bytes of the whole call and of each kernel.

    whole call: read every point once (16 B) + write the dense output,
    V * (16 K + 16) bytes (rows incl. zero padding, 12 B coords, 4 B count).
    insert: its share of the input read, 16 B per prefix point.
    rank:   4 B per prefix point (the slot index written by insert); route 4
            has no rank kernel.
    select: route 4: 16 B per point (every point is read and binned) + one
            4-byte staging word per point of a prefix cell (`staged`);
            otherwise 16 B per point past the prefix + 4 B per prefix point
            (slot), and on the partitioned routes (2, 3) one 4-byte staging
            word per point of a kept pillar (`kept`), route 3 its 16-byte
            row as well.
    pack:   the dense output + 16 B per kept row (gathered from the input, or
            on route 3 copied from the staged rows); the partitioned routes
            also read the staging words back.
    """
    out = V * (16 * K + 16)
    if route == 4:
        return dict(call=16 * N + out, insert=16 * P, rank=0, select=16 * N + 4 * staged,
                    pack=out + 16 * rows + 4 * staged)
    stage = 4 * kept if route >= 2 else 0
    carried = 16 * kept if route == 3 else 0
    return dict(call=16 * N + out, insert=16 * P, rank=4 * P,
                select=16 * (N - P) + 4 * P + stage + carried, pack=out + 16 * rows + stage)


def voxelize_source_hash():
    """sha256 prefix over the sources of the voxelization kernels."""
    import hashlib
    h = hashlib.sha256()
    for f in ("voxelize.hip", "wave_ops.h"):
        h.update(open(os.path.join(ROOT, "sparse_spatial_hashing_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, stage):
    """HBM bytes per launch of the kernel running `stage` from the committed
    counter summary (profiles/<workload>_traffic.txt), or None when it is
    missing or was taken on a different library source than the one built
    now."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = voxelize_source_hash()
    recorded, found = None, None
    for line in open(path):
        if line.startswith("source_sha256:"):
            recorded = line.split(":", 1)[1].strip()
        if line.startswith(f"traffic {stage} "):
            found = int(line.rsplit("bytes=", 1)[1])
    return found if recorded == sha else None


def call_times(vx, x, n, torch):
    """Per-call device times (ms): one pair of HIP events around each call on
    the call's stream, all recorded before one synchronisation."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        vx.run(x)
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def wall_with_readback(vx, x, n, torch):
    """Host wall time per call (ms) including the read-back of V, each call
    finished (one synchronising .item()) before the next starts."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        int(vx.run(x).item())
    return (time.perf_counter() - t0) * 1e3 / n


def staged_points(x, prm, P, vox):
    """Points whose cell holds a prefix point (route 4 stages exactly these),
    counted with the library's own binning step."""
    valid, key = vox.bin_points(x, prm.range_, prm.cell, prm.grid)
    k = key.cpu().numpy()
    v = valid.cpu().numpy()
    head = np.unique(k[:P][v[:P]])
    return int(np.isin(k[v], head).sum())


def time_calls(vx, x, steps, warmup, torch):
    for _ in range(warmup):
        vx.run(x)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        vx.run(x)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def check_parity(vx, pts, prm):
    import oracle
    gv, gc, gn = (t.cpu().numpy() for t in vx.outputs())
    ov, oc, on = oracle.voxelize_params(pts, prm)
    return bool(gv.shape == ov.shape and np.array_equal(gc, oc) and np.array_equal(gn, on)
                and np.array_equal(gv.view(np.uint32), ov.view(np.uint32)))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(pts, prm, seconds):
    """The oracle as it stands, on one host core, repeated on the full cloud
    until `seconds` of CPU work are spent (at least 3 repetitions); beside
    it the NumPy sort-then-segment brute force of the tests (the page's naive
    method), a few repetitions, also one thread."""
    import oracle
    oracle.load()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.voxelize_params(pts, prm)
        reps += 1
        el = time.perf_counter() - t0
        if (el >= seconds and reps >= 3) or reps >= 100000:
            break
    per = el / reps
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from bruteforce import sort_then_segment
    nreps, t1 = 0, time.perf_counter()
    while True:
        sort_then_segment(pts, prm.range_, prm.cell, prm.grid, prm.max_points, prm.max_voxels)
        nreps += 1
        nel = time.perf_counter() - t1
        if (nel >= seconds / 4 and nreps >= 3) or nreps >= 10000:
            break
    nper = nel / nreps
    try:
        aff = sorted(os.sched_getaffinity(0))
    except AttributeError:
        aff = list(range(os.cpu_count() or 1))
    model = cpu_model()
    return {"value": round(pts.shape[0] / per / 1e6, 3), "unit": "Mpoints/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} repetitions of the full {pts.shape[0]:,}-point cloud "
                      f"({el:.1f} s, {per * 1e3:.2f} ms each), single-threaded C oracle, "
                      f"host {model}, {os.cpu_count()} logical CPUs, affinity {len(aff)} CPUs",
            "cpu_model": model, "affinity_cpus": len(aff), "logical_cpus": os.cpu_count(),
            "numpy_bruteforce": {"value": round(pts.shape[0] / nper / 1e6, 3),
                                 "unit": "Mpoints/s", "cores": 1,
                                 "sample": f"{nreps} repetitions of the sort-then-segment "
                                           f"brute force ({nper * 1e3:.1f} ms each)"}}


def run_workload(name, steps, warmup, profile_iters, torch, vox, opts=None):
    from workloads import generate, get_config
    cfg = get_config(name)
    p = cfg.params
    pts, _ = generate(name)
    N = pts.shape[0]
    x = torch.from_numpy(pts).to("cuda:0")
    opts = opts or {}
    vx = vox.Voxelizer(N, p.range_, p.cell, p.grid, p.max_points, p.max_voxels, device="cuda:0",
                       **opts)
    ms = time_calls(vx, x, steps, warmup, torch)
    per_call = call_times(vx, x, steps, torch)
    wall_ms = wall_with_readback(vx, x, max(10, steps // 4), torch)
    vx.run(x)
    torch.cuda.synchronize()
    V = int(vx.num_voxels.item())
    rows = int(vx.num_points[:max(V, 0)].sum().item()) if V > 0 else 0
    parity = check_parity(vx, pts, p)
    stage_ms, total_ms = vx.profile(x, profile_iters)
    pl = vox.plan(N, p.max_voxels, p.max_points, **opts)
    P = pl["prefix_points"]
    route = vox.select_route(N, p.max_voxels, p.max_points, **opts)
    pmap = vox.voxelize(x, p.range_, p.cell, p.grid, p.max_points, p.max_voxels,
                        point_map=True, **opts)[3]
    kept = int((pmap >= 0).sum().item())
    staged = staged_points(x, p, P, vox) if route == 4 else kept
    alg = algorithmic_bytes(N, P, V, p.max_points, rows, kept, staged, route)
    cells = p.grid[0] * p.grid[1] * p.grid[2]
    direct = route == 4 and cells <= 2 * pl["table_slots"] and not opts.get("first_map")
    if route == 4:
        kernels = dict(insert="k_claim" if direct else "k_insert", rank=None,
                       select="k_part_fb", pack="k_bins_fb")
    else:
        kernels = dict(insert="k_insert", rank="k_rank",
                       select="k_part" if route >= 2 else "k_select",
                       pack="k_bins" if route >= 2 else "k_pack")
    timing = {"mean_us": round(ms * 1e3, 2), "median_us": round(float(np.median(per_call)) * 1e3, 2),
              "p10_us": round(float(np.percentile(per_call, 10)) * 1e3, 2),
              "p90_us": round(float(np.percentile(per_call, 90)) * 1e3, 2),
              "wall_us_incl_readback": round(wall_ms * 1e3, 2)}
    return dict(cfg=cfg, pts=pts, N=N, V=V, rows=rows, ms=ms, parity=parity, stage_ms=stage_ms,
                total_ms=total_ms, alg=alg, P=P, kept=kept, staged=staged, kernels=kernels,
                route=route, timing=timing)


# What limits the dominant kernel (the kernel sections of the design notes):
# every voxelization kernel is a chain of dependent memory round trips over
# scattered lines (random cell lookups, short staging runs, row gathers), far
# below HBM bandwidth; its fraction is still stated against the HBM peak.
BOUND = "memory-latency"


def config_line(name, q):
    """One stderr line per workload: time per call, throughput, whole-call
    and dominant-kernel fractions of the HBM peak, parity."""
    stg = {k: v for k, v in q["stage_ms"].items() if q["kernels"][k]}
    dom = max(stg, key=stg.get)
    dom_gbs = q["alg"][dom] / (stg[dom] * 1e-3) / 1e9
    gbs = q["alg"]["call"] / (q["ms"] * 1e-3) / 1e9
    return {"workload": name, "N": q["N"], "V": q["V"], "kept_rows": q["rows"],
            "route": q["route"], **q["timing"],
            "mpoints_s": round(q["N"] / (q["ms"] * 1e-3) / 1e6, 1),
            "gbs_alg": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "dominant": {"kernel": q["kernels"][dom], "us": round(stg[dom] * 1e3, 2),
                         "alg_bytes": int(q["alg"][dom]), "gbs": round(dom_gbs, 1),
                         "frac": round(dom_gbs / HBM_PEAK_GBS, 4)},
            "stages_us": {q["kernels"][k]: round(v * 1e3, 2) for k, v in stg.items()},
            "parity": q["parity"]}


def downsample_line(name, steps, warmup, torch, vox):
    """Voxel-grid downsampling on one workload: µs per call (HIP events on the
    call's stream, inputs resident) and parity with the oracle."""
    import oracle
    from workloads import generate, get_config

    def same_f32(a, b):  # bitwise, except that any NaN equals any NaN
        na, nb = np.isnan(a), np.isnan(b)
        return bool(a.shape == b.shape and np.array_equal(na, nb) and
                    np.array_equal(a.view(np.uint32)[~na], b.view(np.uint32)[~nb]))

    p = get_config(name).params
    pts, _ = generate(name)
    x = torch.from_numpy(pts).to("cuda:0")
    ds = vox.Downsampler(pts.shape[0], p.range_, p.cell, p.grid, p.max_voxels, device="cuda:0")
    ms = time_calls(ds, x, steps, warmup, torch)
    ds.run(x)
    torch.cuda.synchronize()
    got = tuple(t.cpu().numpy() for t in ds.outputs())
    want = oracle.downsample(pts, p.range_, p.cell, p.grid, p.max_voxels)
    ok = (np.array_equal(got[1], want[1]) and np.array_equal(got[2], want[2])
          and same_f32(got[0], want[0]))
    return {"op": "downsample", "workload": name, "N": pts.shape[0], "V": int(got[0].shape[0]),
            "us_per_call": round(ms * 1e3, 2), "mpoints_s": round(pts.shape[0] / (ms * 1e-3) / 1e6, 1),
            "parity": bool(ok)}


def spherical_line(name, steps, warmup, profile_iters, torch, vox):
    """Spherical binning and voxel-contiguous reorder on one workload: µs per
    call (HIP events on the call's stream, inputs resident), per-kernel
    times, algorithmic bytes and parity with the oracle.

    Algorithmic bytes of a call: each point read (16 B) with its voxel id and
    its index in the order written (4 + 4 B); each kept row gathered and
    written in sorted order (16 + 16 B); the voxel offsets (4 B x (voxels + 1))."""
    import oracle
    from workloads import generate, get_sph_config

    p = get_sph_config(name).params
    pts, _ = generate(name)
    x = torch.from_numpy(pts).to("cuda:0")
    s = vox.SphericalSorter(pts.shape[0], p.sph_min, p.sph_cell, p.bins, device="cuda:0")
    ms = time_calls(s, x, steps, warmup, torch)
    stage_ms, total_ms = s.profile(x, profile_iters)
    torch.cuda.synchronize()
    v, off, order, rows = (t.cpu().numpy() for t in s.outputs())
    want = oracle.spherical(pts, p.sph_min, p.sph_cell, p.bins)
    ok = (np.array_equal(v, want[0]) and np.array_equal(off, want[1])
          and np.array_equal(order, want[2])
          and np.array_equal(rows.view(np.uint32), pts[want[2]].view(np.uint32)))
    N, kept, nvox = pts.shape[0], int(order.size), int(np.prod(p.bins))
    # algorithmic bytes of the whole call: read each point, write its voxel id,
    # its index and (kept) row in sorted order, and the voxel offsets
    alg = 16 * N + 4 * N + 4 * N + 32 * kept + 4 * (nvox + 1)
    gbs = alg / (ms * 1e-3) / 1e9
    return {"op": "spherical", "workload": name, "N": N, "kept": kept, "voxels": nvox,
            "us_per_call": round(ms * 1e3, 2),
            "mpoints_s": round(N / (ms * 1e-3) / 1e6, 1),
            "stages_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
            "kernels_us": round(total_ms * 1e3, 2),
            "alg_bytes": alg, "gbs_alg": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "parity": bool(ok)}


def main():
    args = parse()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return
    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Frames are independent, so more GPUs would "
              f"each run their own frames; no cross-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import sparse_spatial_hashing_amd as vox

    opts = json.loads(args.options)
    r = run_workload(args.workload, args.steps, args.warmup, args.profile_iters, torch, vox, opts)
    N, ms = r["N"], r["ms"]
    value = N / (ms * 1e-3) / 1e6
    gbs = r["alg"]["call"] / (ms * 1e-3) / 1e9
    stg = {k: v for k, v in r["stage_ms"].items() if r["kernels"][k]}
    dom = max(stg, key=stg.get)
    dom_ms = stg[dom]
    dom_gbs = r["alg"][dom] / (dom_ms * 1e-3) / 1e9
    p = r["cfg"].params
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "Mpoints/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, **({"options": opts} if opts else {}),
                   "n_points": N, "grid": list(p.grid),
                   "cell_m": list(p.cell), "max_points": p.max_points,
                   "max_voxels": p.max_voxels, "pillars": r["V"], "kept_rows": r["rows"]},
        "achieved_gbs_alg": round(gbs, 1),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "parity_vs_oracle": r["parity"],
        "route": r["route"],
        "timing": r["timing"],
        "stages_ms": {r["kernels"][k]: round(v, 5) for k, v in stg.items()},
        "roofline": {"bound": BOUND, "ceiling": "hbm", "kernel": r["kernels"][dom], "stage": dom,
                     "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "alg_bytes_per_launch": int(r["alg"][dom]),
                     "launch_ms": round(dom_ms, 5),
                     "traffic": recorded_traffic(args.workload, dom)},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(r["pts"], p, args.cpu_seconds)
    if args.all or args.spherical:
        from workloads import sph_config_names
        for name in sph_config_names():
            print(json.dumps(spherical_line(name, args.steps, args.warmup, args.profile_iters,
                                            torch, vox)), file=sys.stderr, flush=True)
    if args.all:
        from workloads import config_names
        for name in config_names():
            print(json.dumps(downsample_line(name, args.steps, args.warmup, torch, vox)),
                  file=sys.stderr, flush=True)
    elif args.downsample:
        print(json.dumps(downsample_line(args.workload, args.steps, args.warmup, torch, vox)),
              file=sys.stderr, flush=True)
    if not args.no_configs:
        from workloads import config_names
        for name in config_names():
            q = r if name == args.workload else run_workload(
                name, args.steps, args.warmup, args.profile_iters, torch, vox)
            print(json.dumps(config_line(name, q)), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
