"""The allocation-free entry point, voxelize_static, against the workspace
entry point voxelize (through the C ABI, bit for bit), on consecutive calls
of different shapes: each call must find its zero part clean although the
library's one scratch array keeps the previous call's contents."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_spatial_hashing_amd as vox  # noqa: E402
from workloads import generate, get_config  # noqa: E402

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def static_call(x, p, K=None, M=None):
    K = p.max_points if K is None else K
    M = p.max_voxels if M is None else M
    out = (torch.full((M, K, 4), 7.0, dtype=torch.float32, device=DEV),
           torch.full((M, 3), -7, dtype=torch.int32, device=DEV),
           torch.full((M,), -7, dtype=torch.int32, device=DEV),
           torch.zeros((1,), dtype=torch.int32, device=DEV))
    rc = vox.voxelize_static(x, p.range_, p.cell, p.grid, K, M, *out)
    assert rc == vox.VOX_OK, vox.strerror(rc)
    torch.cuda.synchronize()
    V = int(out[3].item())
    assert V >= 0, vox.strerror(V)
    return tuple(t[:V].cpu().numpy() for t in out[:3])


def same(a, b, what):
    assert a[0].shape == b[0].shape, (what, a[0].shape, b[0].shape)
    assert np.array_equal(a[1], b[1]), f"{what}: coords differ"
    assert np.array_equal(a[2], b[2]), f"{what}: num_points differ"
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)), f"{what}: voxels differ"


def test_static_entry_matches_workspace_entry_on_consecutive_calls():
    # a large call, then smaller ones (the second call of the pair is
    # smaller), then one whose zero part reaches into the earlier scratch,
    # then the first again
    seq = [("kitti_frame", None), ("tiny", None), ("dense_multisweep", None),
           ("uniform_25k", None), ("voxel3d", None), ("kitti_frame", 20000),
           ("kitti_frame", None)]
    for name, n in seq:
        cfg = get_config(name)
        p = cfg.params
        pts, _ = generate(name, n=n) if n else generate(name)
        say(f"static entry {name} N={pts.shape[0]}")
        x = torch.from_numpy(pts).to(DEV)
        want = tuple(t.cpu().numpy() for t in vox.voxelize(x, p.range_, p.cell, p.grid,
                                                           p.max_points, p.max_voxels))
        got = static_call(x, p)
        same(got, want, f"{name} N={pts.shape[0]}")
        again = static_call(x, p)
        same(again, want, f"{name} N={pts.shape[0]}, repeated")


def test_static_entry_small_then_smaller():
    cfg = get_config("kitti_frame")
    p = cfg.params
    pts, _ = generate("kitti_frame")
    for n in (pts.shape[0], 5000, 0):
        say(f"static entry kitti_frame first {n} points")
        x = torch.from_numpy(np.ascontiguousarray(pts[:n])).to(DEV)
        want = tuple(t.cpu().numpy() for t in vox.voxelize(x, p.range_, p.cell, p.grid,
                                                           p.max_points, p.max_voxels))
        same(static_call(x, p), want, f"first {n}")
