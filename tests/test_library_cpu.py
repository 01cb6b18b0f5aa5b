"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, sizes workspaces, and rejects bad arguments on the host before any
HIP call (so these calls are safe without a GPU)."""
import ctypes
import os
import re

import pytest

import sparse_spatial_hashing_amd as vox

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "voxelize.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("voxelize", "voxelize_ex", "voxelize_chunked", "vox_workspace_bytes",
              "vox_bin_points", "vox_profile_stages", "vox_strerror", "vox_last_hip_error",
              "vox_stage_name", "vox_plan", "voxelize_map"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(vox.LIBRARY_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in voxelize.h but not exported"


def test_library_links_no_oracle():
    data = open(vox.LIBRARY_PATH, "rb").read()
    assert b"oracle_voxelize" not in data and b"oracle_bin" not in data


def test_workspace_bytes_defaults_and_scaling():
    a = vox.workspace_bytes(122880, 12000, 32)
    b = vox.workspace_bytes(2 * 122880, 12000, 32)
    c = vox.workspace_bytes(122880, 24000, 32)
    assert a > 0 and b > a and c > a and a % 256 == 0
    # table 8*M slots of 16 bytes + selection M*K*4 bytes are the big terms
    assert a >= 8 * 12000 * 16 + 12000 * 32 * 4
    assert vox.workspace_bytes(0, 1, 1) > 0


@pytest.mark.parametrize("args", [(-1, 10, 4), (10, 0, 4), (10, 4, 0), (2**30, 10, 4)])
def test_workspace_bytes_rejects_bad_sizes(args):
    with pytest.raises(vox.VoxError):
        vox.workspace_bytes(*args)


def test_workspace_bytes_bucket_cap_option():
    base = vox.workspace_bytes(1000, 100, 32, select_path=1)
    small = vox.workspace_bytes(1000, 100, 32, select_path=1, bucket_cap=64)
    assert small < base          # default bucket is 16 K = 512 slots per pillar
    assert vox.workspace_bytes(1000, 100, 100) > 0   # K > 64 has no bucket
    with pytest.raises(vox.VoxError):
        vox.workspace_bytes(1000, 100, 32, bucket_cap=-1)
    with pytest.raises(vox.VoxError):
        vox.workspace_bytes(1000, 100, 32, bucket_cap=(1 << 20) + 1)


def test_compact_table_option():
    assert vox.workspace_bytes(1000, 100, 32, compact_table=1) > vox.workspace_bytes(1000, 100, 32)
    assert vox.plan(1000, 100, 32)["prefix_points"] == 400   # min(N, 4 * max_voxels)
    with pytest.raises(vox.VoxError):
        vox.workspace_bytes(1000, 100, 32, compact_table=2)


def test_workspace_bytes_rejects_small_table():
    with pytest.raises(vox.VoxError):
        vox.workspace_bytes(1000, 100, 4, table_slots=150)   # needs >= 2 * max_voxels
    assert vox.workspace_bytes(1000, 100, 4, table_slots=200) > 0


def _call(lib, points=0x1000, n=10, rng=(0, -1, -3, 1, 1, 1), cell=(0.1, 0.1, 4), grid=(10, 20, 1),
          K=4, M=8, voxels=0x2000, coords=0x3000, counts=0x4000, nv=0x5000, ws=0x100000,
          wsb=1 << 30):
    r = (ctypes.c_float * 6)(*rng)
    c = (ctypes.c_float * 3)(*cell)
    g = (ctypes.c_int32 * 3)(*grid)
    return lib.voxelize(ctypes.c_void_p(points), n, r, c, g, K, M, ctypes.c_void_p(voxels),
                        ctypes.c_void_p(coords), ctypes.c_void_p(counts), ctypes.c_void_p(nv),
                        ctypes.c_void_p(ws), ctypes.c_size_t(wsb), ctypes.c_void_p(0))


@pytest.mark.parametrize("bad", [
    dict(points=0), dict(points=0x1004), dict(n=-1), dict(rng=(0, -1, -3, 0, 1, 1)),
    dict(rng=(float("nan"), -1, -3, 1, 1, 1)), dict(cell=(0.0, 0.1, 4)),
    dict(cell=(0.1, float("inf"), 4)), dict(grid=(0, 20, 1)), dict(grid=(10, 1 << 25, 1)),
    dict(grid=(1 << 12, 1 << 12, 1 << 9)),
    dict(K=0), dict(M=0), dict(voxels=0), dict(voxels=0x2004), dict(coords=0), dict(counts=0),
    dict(nv=0), dict(ws=0),
])
def test_voxelize_rejects_bad_arguments_on_host(bad):
    assert _call(vox.library(), **bad) == vox.VOX_EINVAL


def test_voxelize_rejects_small_or_misaligned_workspace():
    lib = vox.library()
    need = vox.workspace_bytes(10, 8, 4)
    assert _call(lib, wsb=need - 1) == vox.VOX_EWORKSPACE
    assert _call(lib, ws=0x100010, wsb=need) == vox.VOX_EWORKSPACE


def test_strerror_names_codes():
    for code in (vox.VOX_OK, vox.VOX_EINVAL, vox.VOX_EWORKSPACE, vox.VOX_EHIP,
                 vox.VOX_STATUS_NEEDS_CHUNKED, vox.VOX_STATUS_DEVICE_ERROR):
        assert vox.strerror(code) != "unknown error"
    assert [vox.library().vox_stage_name(k).decode() for k in range(4)] == list(vox.STAGES)


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        vox.voxelize(torch.zeros((4, 4)), (0, 0, 0, 1, 1, 1), (0.1, 0.1, 1), (10, 10, 1), 4, 8)


def test_select_path_option_limits():
    """0 = automatic, 1 = buckets, 2 = partition (K <= 64, max_voxels <= 262144, or
    <= 131072 when K > 32)."""
    auto = vox.workspace_bytes(100000, 60000, 32)
    assert auto == vox.workspace_bytes(100000, 60000, 32, select_path=2)
    assert auto != vox.workspace_bytes(100000, 60000, 32, select_path=1)
    assert vox.plan(100000, 60000, 32)["bucket_cap"] == 0          # no buckets
    assert vox.plan(100000, 60000, 32, select_path=1)["bucket_cap"] == 512
    assert vox.workspace_bytes(1000, 262144, 32, select_path=2) > 0
    # K > 64 or more than 262144 pillars: only the bucket route exists
    assert vox.plan(1000, 100, 65)["bucket_cap"] == 0
    for bad in (dict(select_path=-1), dict(select_path=4)):
        with pytest.raises(vox.VoxError):
            vox.workspace_bytes(1000, 100, 32, **bad)
    assert vox.workspace_bytes(1000, 131072, 64, select_path=2) > 0
    for args in ((1000, 100, 65), (1000, 262145, 32), (1000, 131073, 33)):
        assert vox.workspace_bytes(*args) > 0
        with pytest.raises(vox.VoxError):
            vox.workspace_bytes(*args, select_path=2)
        with pytest.raises(vox.VoxError):
            vox.workspace_bytes(*args, select_path=3)


def test_hash_option_range():
    for h in (0, 1, 2):
        assert vox.workspace_bytes(1000, 100, 32, hash=h) > 0
    for h in (-1, 3):
        with pytest.raises(vox.VoxError):
            vox.workspace_bytes(1000, 100, 32, hash=h)


def test_workspace_zero_part():
    """The zero part precedes the scratch tail; the bucket route has none."""
    for args in ((122880, 12000, 32), (2097152, 60000, 32), (1048576, 40000, 5), (0, 1, 1)):
        total = vox.workspace_bytes(*args)
        zero = vox.workspace_zero_bytes(*args)
        assert 256 <= zero <= total and zero % 256 == 0
        assert vox.workspace_zero_bytes(*args, select_path=1) == \
            vox.workspace_bytes(*args, select_path=1)
    assert vox.workspace_zero_bytes(122880, 12000, 32) < vox.workspace_bytes(122880, 12000, 32)
    with pytest.raises(vox.VoxError):
        vox.workspace_zero_bytes(-1, 12000, 32)


def test_select_route_rules():
    """Automatic route: partitioned with carried rows from 2^19 points up,
    partitioned with gathered rows below, buckets for K > 64."""
    assert vox.select_route(122880, 12000, 32) == 2
    assert vox.select_route(1 << 19, 12000, 32) == 3
    assert vox.select_route(2097152, 60000, 32) == 3
    assert vox.select_route(1000, 100, 65) == 1
    for p in (1, 2, 3):
        assert vox.select_route(122880, 12000, 32, select_path=p) == p
    # carried rows need room for them in the scratch tail
    assert vox.workspace_bytes(122880, 12000, 32, select_path=3) > \
        vox.workspace_bytes(122880, 12000, 32, select_path=2)
    assert vox.workspace_zero_bytes(122880, 12000, 32, select_path=3) == \
        vox.workspace_zero_bytes(122880, 12000, 32, select_path=2)


def test_downsample_workspace_and_limits():
    n, z = vox.downsample_workspace_bytes(122880, 12000)
    assert 256 <= z <= n
    assert vox.downsample_workspace_bytes(122880, 262144)[0] > 0
    for bad in (dict(max_voxels=262145), dict(max_voxels=0)):
        with pytest.raises(vox.VoxError):
            vox.downsample_workspace_bytes(1000, **bad)
    # only the carried-rows route exists for downsampling
    for path in (1, 2):
        with pytest.raises(vox.VoxError):
            vox.downsample_workspace_bytes(1000, 100, select_path=path)
    assert vox.downsample_workspace_bytes(1000, 100, select_path=3)[0] > 0
