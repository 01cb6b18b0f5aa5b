"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, sizes workspaces, and rejects bad arguments on the host before any
HIP call (so these calls are safe without a GPU)."""
import ctypes
import os
import re

import pytest

import sparse_spatial_hashing_amd as vox

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("voxelize", "voxelize_ex", "voxelize_chunked", "vox_workspace_bytes",
              "vox_bin_points", "vox_profile_stages", "vox_strerror", "vox_last_hip_error",
              "vox_stage_name", "vox_plan", "voxelize_map", "sph_table_bytes", "sph_make_table",
              "sph_workspace_bytes", "sph_reorder", "sph_profile_stages", "voxelize_static"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(vox.LIBRARY_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


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
    # the compact table replaces the kept-cell map (which it turns off) and
    # the first-index route (whose direct cell map shares the map's region)
    assert vox.workspace_bytes(1000, 100, 32, compact_table=1) > \
        vox.workspace_bytes(1000, 100, 32, kept_map=1, select_path=2)
    assert vox.select_route(1000, 100, 32, compact_table=1) == 2
    assert vox.plan(1000, 100, 32)["prefix_points"] == 200   # min(N, 2 max_voxels, S/4)
    assert vox.plan(1000, 100, 32, table_slots=400)["prefix_points"] == 100   # S/4
    assert vox.plan(150, 100, 32)["prefix_points"] == 150   # N
    with pytest.raises(vox.VoxError):
        vox.workspace_bytes(1000, 100, 32, compact_table=2)


def test_kept_map_option():
    """The kept-cell map (2 x table_slots cells of 4 bytes) sits in the zero part
    on the partitioned routes; kept_map=1 leaves it out; the bucket route never
    has it."""
    S = vox.plan(122880, 12000, 32)["table_slots"]
    with_map = vox.workspace_zero_bytes(122880, 12000, 32, select_path=2)
    without = vox.workspace_zero_bytes(122880, 12000, 32, select_path=2, kept_map=1)
    assert with_map - without >= 8 * S
    assert vox.workspace_zero_bytes(122880, 12000, 32, select_path=1) == \
        vox.workspace_zero_bytes(122880, 12000, 32, select_path=1, kept_map=1)
    for bad in (-1, 2):
        with pytest.raises(vox.VoxError):
            vox.workspace_bytes(1000, 100, 32, kept_map=bad)


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
    """0 = automatic, 1 = buckets, 2 = partition (K <= 64, max_voxels <= 262144),
    4 = first-index partition (K <= 64, prefix <= 524288 points)."""
    auto = vox.workspace_bytes(100000, 60000, 32)
    assert auto == vox.workspace_bytes(100000, 60000, 32, select_path=4)
    assert vox.select_route(100000, 60000, 32) == 4
    assert auto != vox.workspace_bytes(100000, 60000, 32, select_path=1)
    # the first-index route adds the first occurrences' keys (zero part) and
    # ranks (scratch) to route 2's layout, which the chunked path still uses
    assert auto > vox.workspace_bytes(100000, 60000, 32, select_path=2)
    assert vox.select_route(100000, 60000, 32, select_path=2) == 2
    # bins of 256 slots hold every default prefix the partition admits (at most
    # 2 x 262144 points); a longer prefix leaves route 4 out
    assert vox.select_route(10**6, 262144, 32) == 4
    assert vox.select_route(10**6, 262144, 64) == 4
    assert vox.select_route(10**6, 200000, 32, prefix_points=600000) == 2
    with pytest.raises(vox.VoxError):
        vox.workspace_bytes(10**6, 200000, 32, prefix_points=600000, select_path=4)
    assert vox.plan(100000, 60000, 32)["bucket_cap"] == 0          # no buckets
    assert vox.plan(100000, 60000, 32, select_path=1)["bucket_cap"] == 512
    assert vox.workspace_bytes(1000, 262144, 32, select_path=2) > 0
    # K > 64 or more than 262144 pillars: only the bucket route exists
    assert vox.plan(1000, 100, 65)["bucket_cap"] == 0
    for bad in (dict(select_path=-1), dict(select_path=5), dict(select_path=4, compact_table=1),
                dict(first_map=2), dict(lane_merge=2), dict(bin_ids=8), dict(bin_ids=48),
                dict(bin_ids=512)):
        with pytest.raises(vox.VoxError):
            vox.workspace_bytes(1000, 100, 32, **bad)
    assert vox.select_route(1000, 100, 64, bin_ids=256, select_path=4) == 4
    assert vox.select_route(1000, 100, 32, bin_ids=256) == 4
    assert vox.workspace_bytes(1000, 262144, 64, select_path=2) > 0
    for args in ((1000, 100, 65), (1000, 262145, 32), (1000, 262145, 64)):
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
    """Automatic route: first-index partition with gathered rows, buckets for
    K > 64; pillar-id partition and carried rows only on request."""
    assert vox.select_route(122880, 12000, 32) == 4
    assert vox.select_route(1 << 19, 12000, 32) == 4
    assert vox.select_route(2097152, 60000, 32) == 4
    assert vox.select_route(1048576, 40000, 5) == 4
    assert vox.select_route(1000, 100, 65) == 1
    for p in (1, 2, 3, 4):
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
    # only the carried-rows routes exist for downsampling: 3, and 4 where it
    # applies (its layout holds route 3's too, for the chunked path)
    for path in (1, 2):
        with pytest.raises(vox.VoxError):
            vox.downsample_workspace_bytes(1000, 100, select_path=path)
    n3 = vox.downsample_workspace_bytes(1000, 100, select_path=3)[0]
    n4 = vox.downsample_workspace_bytes(1000, 100, select_path=4)[0]
    assert 0 < n3 < n4 == vox.downsample_workspace_bytes(1000, 100)[0]
    with pytest.raises(vox.VoxError):   # route 4 has no kept-cell table
        vox.downsample_workspace_bytes(1000, 100, select_path=4, compact_table=1)
    # the kept-cell table selects route 3 automatically
    assert vox.downsample_workspace_bytes(1000, 100, compact_table=1)[0] > 0


# ------------------------------------------------------ spherical binning --

SPH_BINS = (16, 18, 72)


def test_sph_table_layout_and_classes():
    """Header fields, and which boundaries lie outside each axis's range: the
    float parameters put boundary 0 of each angle below the range, and the
    last ones (18 and 72) just inside it, so no boundary is above a range."""
    import math
    import struct
    mn, ce = (0.0, -math.pi / 2, -math.pi), (5.0, math.radians(10.0), math.radians(5.0))
    t = vox.sph_table(mn, ce, SPH_BINS)
    assert len(t) == 64 + 8 * (19 + 73)
    h = struct.unpack("<I3i3f3f4i2I", t[:64])
    assert h[1:4] == SPH_BINS
    t_lo, t_hi, p_lo, p_hi = h[10:14]
    a18 = float(ctypes.c_float(-math.pi / 2).value) + 18 * float(ctypes.c_float(ce[1]).value)
    assert a18 < math.pi / 2 and (t_lo, t_hi) == (1, 18)
    a72 = float(ctypes.c_float(-math.pi).value) + 72 * float(ctypes.c_float(ce[2]).value)
    assert a72 < math.pi and (p_lo, p_hi) == (1, 72)
    dirs = struct.unpack(f"<{2 * (19 + 73)}f", t[64:])
    # elevation boundary 9 is at 0 rad to float precision: direction (1, ~0)
    assert dirs[18] == 1.0 and abs(dirs[19]) < 1e-6


@pytest.mark.parametrize("n,bins,opts", [
    (-1, SPH_BINS, {}), (1 << 25, SPH_BINS, {}), (100, (0, 1, 1), {}), (100, (1, 65536, 1), {}),
    (100, (64, 256, 257), {}), (100, SPH_BINS, {"points_per_thread": 3}),
    (100, SPH_BINS, {"digit_bits": 9}), (100, SPH_BINS, {"digit_bits": -1}),
    (100, SPH_BINS, {"sort_tile": 512}), (100, SPH_BINS, {"sort_tile": 3000}),
])
def test_sph_workspace_rejects(n, bins, opts):
    with pytest.raises(vox.VoxError):
        vox.sph_workspace_bytes(n, bins, **opts)


def test_sph_workspace_sizes():
    # two-kernel route (20,736 voxels: 15 key bits): the staging words and rows
    # (20 bytes a point, rounded up to whole tiles) and the (low digit, tile)
    # run words
    a, za = vox.sph_workspace_bytes(65536, SPH_BINS)
    b, zb = vox.sph_workspace_bytes(1 << 20, SPH_BINS)
    assert 65536 * 20 < a < 65536 * 24 and (1 << 20) * 20 < b < (1 << 20) * 24
    # 16 copies of the high-digit counts (8 bits at 2^16 points; 7 at 2^20,
    # where 256 placing blocks keep the look-back short), the error word and
    # the block counter
    assert za == (16 * 256 * 4 + 8 + 255) // 256 * 256
    assert zb == (16 * 128 * 4 + 8 + 255) // 256 * 256
    # radix passes: keys, values and two ping-pong buffers
    c, zc = vox.sph_workspace_bytes(65536, SPH_BINS, digit_bits=8)
    assert 65536 * 12 < c < 65536 * 24
    # 15 key bits as 8 + 7: 16 copies of 256 + 128 counts, and the error word
    assert zc == (16 * 384 * 4 + 4 + 255) // 256 * 256
    assert vox.sph_workspace_bytes(0, SPH_BINS)[0] > 0
    assert vox.sph_workspace_bytes(1 << 24, (64, 256, 256))[0] > 0
    assert vox.sph_workspace_bytes(1 << 24, SPH_BINS)[0] > 0


@pytest.mark.parametrize("bins,digit_bits,kernels", [
    (SPH_BINS, 0, 2), (SPH_BINS, 8, 4), (SPH_BINS, 5, 5), (SPH_BINS, 1, 17),
    ((1, 1, 1), 0, 2), ((1, 1, 1), 8, 3), ((16, 64, 64), 0, 2), ((17, 64, 64), 0, 5),
    ((64, 256, 256), 0, 5), ((64, 256, 256), 1, 25)])
def test_sph_pass_count(bins, digit_bits, kernels):
    """Grids of up to 65,536 voxels take the two-kernel route unless a digit
    width is asked for. Radix keys run over [0, nvox]: 20,736 voxels need 15
    bits (2 passes of 8, 3 of 5, 15 of 1); one voxel needs 1 bit; 69,632
    voxels and 2^22 voxels need 17 and 23 bits (3 passes of 8)."""
    names = vox.sph_stage_names(1000, bins, digit_bits=digit_bits)
    assert len(names) == kernels
    if kernels == 2:
        assert names == ("lowpart", "place")
    else:
        assert names[0] == "key" and names[-1] == "final"


def test_sph_route_limits():
    """The two-kernel route holds up to 2^24 points on a 16-bit grid, also with
    one point per thread (65,536 tiles, split into ranges of 4,096 per placing
    block); a 17-bit grid takes the radix passes."""
    assert len(vox.sph_stage_names(1 << 24, (16, 64, 64))) == 2
    assert len(vox.sph_stage_names(1 << 24, SPH_BINS, points_per_thread=1)) == 2
    assert len(vox.sph_stage_names(1 << 24, (17, 64, 64))) == 5


def test_sph_reorder_rejects_on_host():
    """Argument errors are found before any HIP call."""
    lib = vox.library()
    mn, ce, b = vox._sph_params((0, -1.5, -3.1), (1, 0.1, 0.1), SPH_BINS)
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    base = [fake, 100, mn, ce, b, fake, fake, fake, fake, None, fake, ws, 1 << 30, None, None]
    bad_cell = list(base)
    bad_cell[3] = vox._sph_params((0, 0, 0), (1, 0.0, 0.1), SPH_BINS)[1]
    assert lib.sph_reorder(*bad_cell) == vox.VOX_EINVAL
    no_table = list(base)
    no_table[5] = None
    assert lib.sph_reorder(*no_table) == vox.VOX_EINVAL
    small = list(base)
    small[12] = 16
    assert lib.sph_reorder(*small) == vox.VOX_EWORKSPACE
    odd = list(base)
    odd[0] = ctypes.c_void_p((1 << 20) + 4)
    assert lib.sph_reorder(*odd) == vox.VOX_EINVAL
    assert "boundary table" in vox.strerror(vox.SPH_STATUS_BAD_TABLE)


def test_voxelize_map_chunked_mode_range():
    """voxelize_map's chunked argument: 0 single pass, 1 chunked, 2 automatic;
    anything else is rejected on the host before any HIP call."""
    lib = vox.library()
    r = (ctypes.c_float * 6)(0, -1, -3, 1, 1, 1)
    c = (ctypes.c_float * 3)(0.1, 0.1, 4)
    g = (ctypes.c_int32 * 3)(10, 20, 1)
    for bad in (-1, 3):
        rc = lib.voxelize_map(ctypes.c_void_p(0x1000), 10, r, c, g, 4, 8, ctypes.c_void_p(0x2000),
                              ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000),
                              ctypes.c_void_p(0x5000), None, ctypes.c_void_p(0x100000),
                              ctypes.c_size_t(1 << 30), None, None, bad)
        assert rc == vox.VOX_EINVAL


def test_voxelize_static_size_limit_rejected_on_host():
    """The allocation-free entry point refuses a call whose layout exceeds its
    64 MiB array with VOX_ESCRATCH, and bad arguments with VOX_EINVAL, before
    any HIP call (so this runs without a GPU)."""
    lib = vox.library()
    r = (ctypes.c_float * 6)(0, -40, -3, 70, 40, 1)
    c = (ctypes.c_float * 3)(0.1, 0.1, 4)
    g = (ctypes.c_int32 * 3)(700, 800, 1)
    n, M, K = 20_000_000, 60000, 32
    assert vox.workspace_bytes(n, M, K) > (64 << 20)
    args = [ctypes.c_void_p(0x1000), n, r, c, g, K, M, ctypes.c_void_p(0x2000),
            ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000), None]
    assert lib.voxelize_static(*args) == vox.VOX_ESCRATCH
    assert "scratch" in vox.strerror(vox.VOX_ESCRATCH)
    args[7] = None  # null output
    assert lib.voxelize_static(*args) == vox.VOX_EINVAL
