"""MI355X (gfx950) pillar / voxel binning: a thin ctypes binding over libvoxelize.so.

Every step of the operation runs in the library's HIP kernels; this module
only checks tensor arguments (dtype, device, contiguity), allocates outputs
and the workspace with torch, passes raw pointers and the current stream, and
reads the pillar count back (one synchronisation), as the "Voxelize" page's
Python entry point does ("The PyTorch side"). There is no CPU fallback: if the
library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Optional, Sequence, Tuple

import torch  # imported first: the library binds to the HIP runtime torch has loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libvoxelize.so")

VOX_OK = 0
VOX_EINVAL = -1
VOX_EWORKSPACE = -2
VOX_EHIP = -4
VOX_ESCRATCH = -5
VOX_STATUS_NEEDS_CHUNKED = -16
VOX_STATUS_DEVICE_ERROR = -17
SPH_STATUS_BAD_TABLE = -18
STAGES = ("insert", "rank", "select", "pack")
HEADER_BYTES = 256          # the workspace's first 256 bytes hold the result words


def workspace_is_clean(ws: "torch.Tensor", zero_bytes: Optional[int] = None) -> bool:
    """True when a workspace is ready for reuse by a call whose zero part is
    `zero_bytes` long (default: the whole workspace): the zero part past the
    header is zero and so are the header's counters (only the two result
    words, bytes 8..16, may be nonzero)."""
    end = ws.numel() if zero_bytes is None else int(zero_bytes)
    head = ws[:HEADER_BYTES].view(torch.int32)
    rest_zero = int(torch.count_nonzero(ws[HEADER_BYTES:end]).item()) == 0
    counters = torch.cat([head[0:2], head[4:]])
    return rest_zero and int(torch.count_nonzero(counters).item()) == 0


class VoxError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class Options(ctypes.Structure):
    """Mirror of ``vox_options`` (0 fields mean defaults)."""
    _fields_ = [("table_slots", ctypes.c_int64), ("prefix_points", ctypes.c_int64),
                ("hash", ctypes.c_int32), ("bucket_cap", ctypes.c_int32),
                ("compact_table", ctypes.c_int32), ("select_path", ctypes.c_int32),
                ("kept_map", ctypes.c_int32), ("first_map", ctypes.c_int32),
                ("lane_merge", ctypes.c_int32), ("bin_ids", ctypes.c_int32)]


class SphOptions(ctypes.Structure):
    _fields_ = [("points_per_thread", ctypes.c_int32), ("digit_bits", ctypes.c_int32),
                ("sort_tile", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(
            f"{LIBRARY_PATH} is missing: build it with `python sparse_spatial_hashing_amd/csrc/build.py`"
            " (there is no CPU fallback)")
    lib = ctypes.CDLL(LIBRARY_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    op = ctypes.POINTER(Options)
    lib.vox_workspace_bytes.argtypes = [i64, i32, i32, op]
    lib.vox_workspace_bytes.restype = i64
    lib.vox_workspace_zero_bytes.argtypes = [i64, i32, i32, op]
    lib.vox_workspace_zero_bytes.restype = i64
    lib.vox_select_route.argtypes = [i64, i32, i32, op]
    lib.vox_select_route.restype = i32
    lib.vox_downsample_workspace_bytes.argtypes = [i64, i32, op]
    lib.vox_downsample_workspace_bytes.restype = i64
    lib.vox_downsample_workspace_zero_bytes.argtypes = [i64, i32, op]
    lib.vox_downsample_workspace_zero_bytes.restype = i64
    lib.vox_downsample.argtypes = [vp, i64, vp, vp, vp, i32, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                   vp, op, i32]
    lib.vox_downsample.restype = ctypes.c_int
    common = [vp, i64, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.voxelize.argtypes = common
    lib.voxelize.restype = ctypes.c_int
    for name in ("voxelize_ex", "voxelize_chunked"):
        f = getattr(lib, name)
        f.argtypes = common + [op]
        f.restype = ctypes.c_int
    lib.voxelize_map.argtypes = [vp, i64, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp,
                                 op, i32]
    lib.voxelize_map.restype = ctypes.c_int
    lib.voxelize_static.argtypes = [vp, i64, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.voxelize_static.restype = ctypes.c_int
    lib.vox_plan.argtypes = [i64, i32, i32, op, vp, vp, vp]
    lib.vox_plan.restype = ctypes.c_int
    lib.vox_bin_points.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp]
    lib.vox_bin_points.restype = ctypes.c_int
    lib.vox_profile_stages.argtypes = common + [op, i32, vp, vp]
    lib.vox_profile_stages.restype = ctypes.c_int
    sop = ctypes.POINTER(SphOptions)
    lib.sph_table_bytes.argtypes = [vp]
    lib.sph_table_bytes.restype = i64
    lib.sph_make_table.argtypes = [vp, vp, vp, vp, i64]
    lib.sph_make_table.restype = ctypes.c_int
    lib.sph_workspace_bytes.argtypes = [i64, vp, sop]
    lib.sph_workspace_bytes.restype = i64
    lib.sph_workspace_zero_bytes.argtypes = [i64, vp, sop]
    lib.sph_workspace_zero_bytes.restype = i64
    lib.sph_num_kernels.argtypes = [i64, vp, sop]
    lib.sph_num_kernels.restype = i32
    sph_common = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, sop, vp]
    lib.sph_reorder.argtypes = sph_common
    lib.sph_reorder.restype = ctypes.c_int
    lib.sph_profile_stages.argtypes = sph_common + [i32, vp, vp]
    lib.sph_profile_stages.restype = ctypes.c_int
    lib.vox_stage_name.argtypes = [i32]
    lib.vox_stage_name.restype = ctypes.c_char_p
    lib.vox_strerror.argtypes = [i32]
    lib.vox_strerror.restype = ctypes.c_char_p
    lib.vox_last_hip_error.argtypes = []
    lib.vox_last_hip_error.restype = i32
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def strerror(code: int) -> str:
    return _lib.vox_strerror(int(code)).decode()


def _check(rc: int, what: str) -> None:
    if rc != VOX_OK:
        if rc == VOX_EHIP:
            raise VoxError(rc, f"{what} (hipError {_lib.vox_last_hip_error()})")
        raise VoxError(rc, what)


def _options(table_slots: int = 0, prefix_points: int = 0, hash: int = 0, bucket_cap: int = 0,
             compact_table: int = 0, select_path: int = 0, kept_map: int = 0, first_map: int = 0,
             lane_merge: int = 0, bin_ids: int = 0):
    vals = (table_slots, prefix_points, hash, bucket_cap, compact_table, select_path, kept_map,
            first_map, lane_merge, bin_ids)
    if not any(vals):
        return None
    return ctypes.pointer(Options(*[int(v) for v in vals]))


def workspace_bytes(n_points: int, max_voxels: int, max_points: int, **opts) -> int:
    n = _lib.vox_workspace_bytes(int(n_points), int(max_voxels), int(max_points), _options(**opts))
    if n < 0:
        raise VoxError(int(n), "vox_workspace_bytes")
    return int(n)


def select_route(n_points: int, max_voxels: int, max_points: int, **opts) -> int:
    """The route a single-pass call takes: 1 buckets, 2 partitioned by pillar id
    (rows gathered from the cloud), 3 as 2 with rows carried through scratch,
    4 partitioned by first index (no rank kernel)."""
    r = _lib.vox_select_route(int(n_points), int(max_voxels), int(max_points), _options(**opts))
    if r < 0:
        raise VoxError(int(r), "vox_select_route")
    return int(r)


def workspace_zero_bytes(n_points: int, max_voxels: int, max_points: int, **opts) -> int:
    """Bytes at the start of the workspace that must be zero before a call
    (and are zero again after it); the rest is scratch."""
    n = _lib.vox_workspace_zero_bytes(int(n_points), int(max_voxels), int(max_points),
                                      _options(**opts))
    if n < 0:
        raise VoxError(int(n), "vox_workspace_zero_bytes")
    return int(n)


def plan(n_points: int, max_voxels: int, max_points: int, **opts) -> Dict[str, int]:
    """Table slots, prefix length and bucket slots a call with these sizes uses."""
    S, P, cap = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(_lib.vox_plan(int(n_points), int(max_voxels), int(max_points), _options(**opts),
                         ctypes.byref(S), ctypes.byref(P), ctypes.byref(cap)), "vox_plan")
    return {"table_slots": S.value, "prefix_points": P.value, "bucket_cap": cap.value}


class _Workspaces:
    """Workspaces reused per (device, stream). A completed call leaves the
    zero part of its own layout zero and may leave scratch after it; the cache
    remembers how long the zero prefix is and clears, on the call's stream,
    only what a larger zero part of the next call adds. A workspace that saw
    a device error is dropped."""

    def __init__(self):
        self._lock = threading.Lock()
        self._cache: Dict[Tuple[int, int], torch.Tensor] = {}
        self._clean: Dict[Tuple[int, int], int] = {}

    def get(self, device: torch.device, stream: int, nbytes: int,
            zero_bytes: int) -> torch.Tensor:
        key = (device.index, stream)
        with self._lock:
            ws = self._cache.get(key)
            if ws is None or ws.numel() < nbytes:
                ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
                self._cache[key] = ws
                self._clean[key] = ws.numel()
            clean = self._clean[key]
            if clean < zero_bytes:
                ws[clean:zero_bytes].zero_()  # scratch of an earlier, smaller layout
            # the call will leave [0, zero_bytes) zero and use the rest as scratch
            self._clean[key] = zero_bytes
            return ws

    def drop(self, device: torch.device, stream: int) -> None:
        with self._lock:
            self._cache.pop((device.index, stream), None)
            self._clean.pop((device.index, stream), None)


_workspaces = _Workspaces()


def _host_params(range_, cell, grid):
    r = (ctypes.c_float * 6)(*[float(v) for v in range_])
    c = (ctypes.c_float * 3)(*[float(v) for v in cell])
    g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    return r, c, g


def _check_points(points: torch.Tensor) -> None:
    if not isinstance(points, torch.Tensor):
        raise TypeError("points must be a torch.Tensor")
    if points.dtype != torch.float32 or points.dim() != 2 or points.shape[1] != 4:
        raise ValueError("points must be a [N, 4] float32 tensor")
    if not points.is_cuda:
        raise ValueError("points must be on a GPU device")
    if not points.is_contiguous():
        raise ValueError("points must be contiguous")


@torch.no_grad()
def voxelize(points: torch.Tensor, range_: Sequence[float], cell: Sequence[float],
             grid: Sequence[int], max_points: int, max_voxels: int, *,
             table_slots: int = 0, prefix_points: int = 0, hash: int = 0, bucket_cap: int = 0,
             compact_table: int = 0, select_path: int = 0, kept_map: int = 0,
             first_map: int = 0, lane_merge: int = 0, bin_ids: int = 0,
             chunked: bool = False, point_map: bool = False,
             return_device_outputs: bool = False):
    """Pillar / voxel binning of one [N, 4] float32 cloud on the GPU.

    Returns ``(voxels[V, K, 4] f32, coords[V, 3] i32 (z, y, x), num_points[V] i32)``
    as views of freshly allocated outputs, and with ``point_map=True`` also
    ``point_pillar[N] i32`` (pillar id of each point's cell when kept, else -1).
    ``chunked=True`` calls the chunked path directly; otherwise the library's
    automatic mode runs the single pass and takes the chunked path only when
    the single pass reports that the cap could not be decided.
    """
    _check_points(points)
    dev = points.device
    N, K, M = points.shape[0], int(max_points), int(max_voxels)
    kw = dict(table_slots=table_slots, prefix_points=prefix_points, hash=hash,
              bucket_cap=bucket_cap, compact_table=compact_table, select_path=select_path,
              kept_map=kept_map, first_map=first_map, lane_merge=lane_merge, bin_ids=bin_ids)
    opts = _options(**kw)
    nbytes = workspace_bytes(N, M, K, **kw)
    zbytes = workspace_zero_bytes(N, M, K, **kw)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        ws = _workspaces.get(dev, stream, nbytes, zbytes)
        voxels = torch.empty((M, K, 4), dtype=torch.float32, device=dev)
        coords = torch.empty((M, 3), dtype=torch.int32, device=dev)
        counts = torch.empty((M,), dtype=torch.int32, device=dev)
        nv = torch.empty((1,), dtype=torch.int32, device=dev)
        pmap = torch.empty((N,), dtype=torch.int32, device=dev) if point_map else None
        r, c, g = _host_params(range_, cell, grid)
        args = [ctypes.c_void_p(points.data_ptr()), N, r, c, g, K, M,
                ctypes.c_void_p(voxels.data_ptr()), ctypes.c_void_p(coords.data_ptr()),
                ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(nv.data_ptr()),
                ctypes.c_void_p(pmap.data_ptr() if pmap is not None else 0),
                ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                ctypes.c_void_p(stream), opts]
        rc = _lib.voxelize_map(*args, 1 if chunked else 2)
        if rc not in (VOX_OK, VOX_EINVAL, VOX_EWORKSPACE):
            _workspaces.drop(dev, stream)  # kernels may have run: the workspace may be dirty
        _check(rc, "voxelize")
        V = int(nv.item())
        if V < 0:
            _workspaces.drop(dev, stream)
            raise VoxError(V, "voxelize (device status)")
    if return_device_outputs:
        return voxels, coords, counts, nv
    if point_map:
        return voxels[:V], coords[:V], counts[:V], pmap
    return voxels[:V], coords[:V], counts[:V]


@torch.no_grad()
def voxelize_static(points: torch.Tensor, range_: Sequence[float], cell: Sequence[float],
                    grid: Sequence[int], max_points: int, max_voxels: int,
                    voxels: torch.Tensor, coords: torch.Tensor, num_points: torch.Tensor,
                    num_voxels: torch.Tensor) -> int:
    """The library's allocation-free entry point: one call into caller-owned
    outputs (voxels [M,K,4] f32, coords [M,3] i32, num_points [M] i32,
    num_voxels [1] i32, all on the points' device), with the library's own
    per-GPU scratch array as the workspace. Enqueued on the current stream;
    nothing is allocated and nothing synchronised. Returns the C return code
    (VOX_OK, or VOX_ESCRATCH when the call needs more than the array)."""
    _check_points(points)
    dev = points.device
    N, K, M = points.shape[0], int(max_points), int(max_voxels)
    for t, shape, dt in ((voxels, (M, K, 4), torch.float32), (coords, (M, 3), torch.int32),
                         (num_points, (M,), torch.int32), (num_voxels, (1,), torch.int32)):
        if t.device != dev or tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"output must be a contiguous {dt} tensor of shape {shape} on {dev}")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        r, c, g = _host_params(range_, cell, grid)
        rc = _lib.voxelize_static(ctypes.c_void_p(points.data_ptr()), N, r, c, g, K, M,
                                  ctypes.c_void_p(voxels.data_ptr()),
                                  ctypes.c_void_p(coords.data_ptr()),
                                  ctypes.c_void_p(num_points.data_ptr()),
                                  ctypes.c_void_p(num_voxels.data_ptr()), ctypes.c_void_p(stream))
    if rc not in (VOX_OK, VOX_ESCRATCH):
        _check(rc, "voxelize_static")
    return int(rc)


def downsample_workspace_bytes(n_points: int, max_voxels: int, **opts) -> Tuple[int, int]:
    """(workspace bytes, bytes of its zero part) for vox_downsample."""
    o = _options(**opts)
    n = _lib.vox_downsample_workspace_bytes(int(n_points), int(max_voxels), o)
    z = _lib.vox_downsample_workspace_zero_bytes(int(n_points), int(max_voxels), o)
    if n < 0 or z < 0:
        raise VoxError(int(min(n, z)), "vox_downsample_workspace_bytes")
    return int(n), int(z)


@torch.no_grad()
def downsample(points: torch.Tensor, range_: Sequence[float], cell: Sequence[float],
               grid: Sequence[int], max_voxels: int, *, table_slots: int = 0,
               prefix_points: int = 0, hash: int = 0, compact_table: int = 0, kept_map: int = 0,
               select_path: int = 0, first_map: int = 0, lane_merge: int = 0, bin_ids: int = 0,
               chunked: bool = False):
    """Voxel-grid downsampling: (centroids [V,4] f32 (x, y, z, intensity means),
    coords [V,3] i32 (z, y, x), counts [V] i32) for the first max_voxels voxels
    in first-occurrence order. select_path 0 (automatic: the first-index
    route where it applies, else 3), 3 or 4. The chunked route is taken when
    the single pass reports that the cap could not be decided."""
    _check_points(points)
    dev = points.device
    N, M = points.shape[0], int(max_voxels)
    kw = dict(table_slots=table_slots, prefix_points=prefix_points, hash=hash,
              compact_table=compact_table, kept_map=kept_map, select_path=select_path,
              first_map=first_map, lane_merge=lane_merge, bin_ids=bin_ids)
    opts = _options(**kw)
    nbytes, zbytes = downsample_workspace_bytes(N, M, **kw)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        ws = _workspaces.get(dev, stream, nbytes, zbytes)
        cen = torch.empty((M, 4), dtype=torch.float32, device=dev)
        coords = torch.empty((M, 3), dtype=torch.int32, device=dev)
        counts = torch.empty((M,), dtype=torch.int32, device=dev)
        nv = torch.empty((1,), dtype=torch.int32, device=dev)
        r, c, g = _host_params(range_, cell, grid)
        args = [ctypes.c_void_p(points.data_ptr()), N, r, c, g, M,
                ctypes.c_void_p(cen.data_ptr()), ctypes.c_void_p(coords.data_ptr()),
                ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(nv.data_ptr()),
                ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                ctypes.c_void_p(stream), opts]
        rc = _lib.vox_downsample(*args, 1 if chunked else 0)
        if rc not in (VOX_OK, VOX_EINVAL, VOX_EWORKSPACE):
            _workspaces.drop(dev, stream)  # kernels may have run: the workspace may be dirty
        _check(rc, "vox_downsample")
        V = int(nv.item())
        if V == VOX_STATUS_NEEDS_CHUNKED and not chunked:
            rc = _lib.vox_downsample(*args, 1)
            if rc not in (VOX_OK, VOX_EINVAL, VOX_EWORKSPACE):
                _workspaces.drop(dev, stream)
            _check(rc, "vox_downsample (chunked)")
            V = int(nv.item())
        if V < 0:
            _workspaces.drop(dev, stream)
            raise VoxError(V, "vox_downsample (device status)")
    return cen[:V], coords[:V], counts[:V]


@torch.no_grad()
def bin_points(points: torch.Tensor, range_: Sequence[float], cell: Sequence[float],
               grid: Sequence[int]) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-point binning alone: (valid bool[N], key int64[N], -1 when rejected)."""
    _check_points(points)
    dev = points.device
    N = points.shape[0]
    with torch.cuda.device(dev):
        valid = torch.empty((N,), dtype=torch.int8, device=dev)
        key = torch.empty((N,), dtype=torch.int64, device=dev)
        r, c, g = _host_params(range_, cell, grid)
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(_lib.vox_bin_points(ctypes.c_void_p(points.data_ptr()), N, r, c, g,
                                   ctypes.c_void_p(valid.data_ptr()),
                                   ctypes.c_void_p(key.data_ptr()), ctypes.c_void_p(stream)),
               "vox_bin_points")
    return valid.bool(), key


class Voxelizer:
    """Pre-allocated outputs and workspace for repeated calls with one shape.

    ``run(points)`` enqueues one call on the current stream and returns the
    device tensor holding V; nothing is allocated or synchronised per call.
    Used by the benchmark and by callers that keep their own stream timing.
    """

    def __init__(self, n_points: int, range_, cell, grid, max_points: int, max_voxels: int,
                 device="cuda", **opts):
        self.N, self.K, self.M = int(n_points), int(max_points), int(max_voxels)
        self.device = torch.device(device)
        self._opts = _options(**opts)
        self.nbytes = workspace_bytes(self.N, self.M, self.K, **opts)
        self.zero_bytes = workspace_zero_bytes(self.N, self.M, self.K, **opts)
        self.workspace = torch.zeros(self.nbytes, dtype=torch.uint8, device=self.device)
        self.voxels = torch.empty((self.M, self.K, 4), dtype=torch.float32, device=self.device)
        self.coords = torch.empty((self.M, 3), dtype=torch.int32, device=self.device)
        self.num_points = torch.empty((self.M,), dtype=torch.int32, device=self.device)
        self.num_voxels = torch.zeros((1,), dtype=torch.int32, device=self.device)
        self._r, self._c, self._g = _host_params(range_, cell, grid)

    def _args(self, points: torch.Tensor, stream: int):
        _check_points(points)
        if points.shape[0] != self.N:
            raise ValueError(f"expected {self.N} points, got {points.shape[0]}")
        return [ctypes.c_void_p(points.data_ptr()), self.N, self._r, self._c, self._g, self.K,
                self.M, ctypes.c_void_p(self.voxels.data_ptr()),
                ctypes.c_void_p(self.coords.data_ptr()),
                ctypes.c_void_p(self.num_points.data_ptr()),
                ctypes.c_void_p(self.num_voxels.data_ptr()),
                ctypes.c_void_p(self.workspace.data_ptr()), ctypes.c_size_t(self.nbytes),
                ctypes.c_void_p(stream)]

    def run(self, points: torch.Tensor) -> torch.Tensor:
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _check(_lib.voxelize_ex(*self._args(points, stream), self._opts), "voxelize")
        return self.num_voxels

    def profile(self, points: torch.Tensor, iters: int) -> Tuple[Dict[str, float], float]:
        """Mean milliseconds per stage and per call, from HIP events on the call's stream."""
        stream = torch.cuda.current_stream(self.device).cuda_stream
        stage = (ctypes.c_float * len(STAGES))()
        total = ctypes.c_float()
        _check(_lib.vox_profile_stages(*self._args(points, stream), self._opts, int(iters),
                                       stage, ctypes.byref(total)), "vox_profile_stages")
        return {STAGES[k]: float(stage[k]) for k in range(len(STAGES))}, float(total.value)

    def outputs(self):
        V = int(self.num_voxels.item())
        if V < 0:
            raise VoxError(V, "voxelize (device status)")
        return self.voxels[:V], self.coords[:V], self.num_points[:V]


class Downsampler:
    """Pre-allocated outputs and workspace for repeated voxel-grid
    downsampling calls with one shape; ``run(points)`` enqueues one call on
    the current stream (nothing allocated or synchronised per call)."""

    def __init__(self, n_points: int, range_, cell, grid, max_voxels: int, device="cuda",
                 **opts):
        self.N, self.M = int(n_points), int(max_voxels)
        self.device = torch.device(device)
        self._opts = _options(**opts)
        self.nbytes, self.zero_bytes = downsample_workspace_bytes(self.N, self.M, **opts)
        self.workspace = torch.zeros(self.nbytes, dtype=torch.uint8, device=self.device)
        self.centroids = torch.empty((self.M, 4), dtype=torch.float32, device=self.device)
        self.coords = torch.empty((self.M, 3), dtype=torch.int32, device=self.device)
        self.counts = torch.empty((self.M,), dtype=torch.int32, device=self.device)
        self.num_voxels = torch.zeros((1,), dtype=torch.int32, device=self.device)
        self._r, self._c, self._g = _host_params(range_, cell, grid)

    def run(self, points: torch.Tensor) -> torch.Tensor:
        _check_points(points)
        if points.shape[0] != self.N:
            raise ValueError(f"expected {self.N} points, got {points.shape[0]}")
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _check(_lib.vox_downsample(
            ctypes.c_void_p(points.data_ptr()), self.N, self._r, self._c, self._g, self.M,
            ctypes.c_void_p(self.centroids.data_ptr()), ctypes.c_void_p(self.coords.data_ptr()),
            ctypes.c_void_p(self.counts.data_ptr()), ctypes.c_void_p(self.num_voxels.data_ptr()),
            ctypes.c_void_p(self.workspace.data_ptr()), ctypes.c_size_t(self.nbytes),
            ctypes.c_void_p(stream), self._opts, 0), "vox_downsample")
        return self.num_voxels

    def outputs(self):
        V = int(self.num_voxels.item())
        if V < 0:
            raise VoxError(V, "vox_downsample (device status)")
        return self.centroids[:V], self.coords[:V], self.counts[:V]


# ------------------------------------------------------ spherical binning --

def _sph_params(sph_min, sph_cell, bins):
    mn = (ctypes.c_float * 3)(*[float(v) for v in sph_min])
    ce = (ctypes.c_float * 3)(*[float(v) for v in sph_cell])
    b = (ctypes.c_int32 * 3)(*[int(v) for v in bins])
    return mn, ce, b


def _sph_options(points_per_thread: int = 0, digit_bits: int = 0, sort_tile: int = 0):
    if not (points_per_thread or digit_bits or sort_tile):
        return None
    return ctypes.pointer(SphOptions(int(points_per_thread), int(digit_bits), int(sort_tile)))


def sph_table(sph_min: Sequence[float], sph_cell: Sequence[float],
              bins: Sequence[int]) -> bytes:
    """The boundary table of these parameters (host bytes, from sph_make_table)."""
    mn, ce, b = _sph_params(sph_min, sph_cell, bins)
    n = _lib.sph_table_bytes(b)
    if n < 0:
        raise VoxError(int(n), "sph_table_bytes")
    buf = (ctypes.c_uint8 * int(n))()
    _check(_lib.sph_make_table(mn, ce, b, buf, int(n)), "sph_make_table")
    return bytes(buf)


class _SphTables:
    """Device copies of boundary tables, one per (device, parameters); each is
    made once (one host-to-device copy) and kept."""

    def __init__(self):
        self._lock = threading.Lock()
        self._cache: Dict[Tuple, torch.Tensor] = {}

    def get(self, device: torch.device, sph_min, sph_cell, bins) -> torch.Tensor:
        f32 = lambda v: ctypes.c_float(float(v)).value  # noqa: E731  (float32 rounding)
        key = (device.index, tuple(f32(v) for v in sph_min), tuple(f32(v) for v in sph_cell),
               tuple(int(v) for v in bins))
        with self._lock:
            t = self._cache.get(key)
            if t is None:
                host = torch.frombuffer(bytearray(sph_table(sph_min, sph_cell, bins)),
                                        dtype=torch.uint8)
                t = host.to(device)
                self._cache[key] = t
            return t


_sph_tables = _SphTables()


def sph_workspace_bytes(n_points: int, bins: Sequence[int], **opts) -> Tuple[int, int]:
    """(workspace bytes, bytes of its zero part) for sph_reorder."""
    b = (ctypes.c_int32 * 3)(*[int(v) for v in bins])
    o = _sph_options(**opts)
    n = _lib.sph_workspace_bytes(int(n_points), b, o)
    z = _lib.sph_workspace_zero_bytes(int(n_points), b, o)
    if n < 0 or z < 0:
        raise VoxError(int(min(n, z)), "sph_workspace_bytes")
    return int(n), int(z)


def sph_stage_names(n_points: int, bins: Sequence[int], **opts) -> Tuple[str, ...]:
    """Names of the kernels one call launches, in order: (lowpart, place) on the
    two-kernel route (keys of at most 16 bits), else key, pass0.., final."""
    b = (ctypes.c_int32 * 3)(*[int(v) for v in bins])
    k = _lib.sph_num_kernels(int(n_points), b, _sph_options(**opts))
    if k < 0:
        raise VoxError(int(k), "sph_num_kernels")
    if k == 2:
        return ("lowpart", "place")
    return ("key",) + tuple(f"pass{q}" for q in range(k - 2)) + ("final",)


class SphericalSorter:
    """Pre-allocated outputs and workspace for repeated spherical binning and
    reorder calls with one shape; ``run(points)`` enqueues one call on the
    current stream (nothing allocated or synchronised per call)."""

    def __init__(self, n_points: int, sph_min, sph_cell, bins, device="cuda", sorted_rows=True,
                 **opts):
        self.N = int(n_points)
        self.device = torch.device(device)
        self.bins = tuple(int(v) for v in bins)
        self.nvox = self.bins[0] * self.bins[1] * self.bins[2]
        self._opts = _sph_options(**opts)
        self._mn, self._ce, self._b = _sph_params(sph_min, sph_cell, bins)
        self.table = _sph_tables.get(self.device, sph_min, sph_cell, bins)
        self.nbytes, self.zero_bytes = sph_workspace_bytes(self.N, bins, **opts)
        self.stages = sph_stage_names(self.N, bins, **opts)
        # the zero part must be zero before the first call; each call leaves it so
        self.workspace = torch.zeros(max(self.nbytes, 256), dtype=torch.uint8, device=self.device)
        self.voxel_of = torch.empty((self.N,), dtype=torch.int32, device=self.device)
        self.offsets = torch.empty((self.nvox + 1,), dtype=torch.int32, device=self.device)
        self.order = torch.empty((max(self.N, 1),), dtype=torch.int32, device=self.device)
        self.sorted = (torch.empty((max(self.N, 1), 4), dtype=torch.float32, device=self.device)
                       if sorted_rows else None)
        self.n_kept = torch.zeros((1,), dtype=torch.int32, device=self.device)

    def _args(self, points: torch.Tensor, stream: int):
        _check_points(points)
        if points.shape[0] != self.N:
            raise ValueError(f"expected {self.N} points, got {points.shape[0]}")
        if points.device != self.device:
            raise ValueError(f"points are on {points.device}, the sorter on {self.device}")
        return [ctypes.c_void_p(points.data_ptr()), self.N, self._mn, self._ce, self._b,
                ctypes.c_void_p(self.table.data_ptr()), ctypes.c_void_p(self.voxel_of.data_ptr()),
                ctypes.c_void_p(self.offsets.data_ptr()), ctypes.c_void_p(self.order.data_ptr()),
                ctypes.c_void_p(self.sorted.data_ptr()) if self.sorted is not None else None,
                ctypes.c_void_p(self.n_kept.data_ptr()), ctypes.c_void_p(self.workspace.data_ptr()),
                self.nbytes, self._opts, ctypes.c_void_p(stream)]

    def run(self, points: torch.Tensor) -> torch.Tensor:
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _check(_lib.sph_reorder(*self._args(points, stream)), "sph_reorder")
        return self.n_kept

    def profile(self, points: torch.Tensor, iters: int) -> Tuple[Dict[str, float], float]:
        """Mean milliseconds per kernel and per call, from HIP events on the call's stream."""
        stream = torch.cuda.current_stream(self.device).cuda_stream
        stage = (ctypes.c_float * len(self.stages))()
        total = ctypes.c_float()
        _check(_lib.sph_profile_stages(*self._args(points, stream), int(iters), stage,
                                       ctypes.byref(total)), "sph_profile_stages")
        return {name: float(stage[k]) for k, name in enumerate(self.stages)}, float(total.value)

    def outputs(self):
        """(voxel_of [N], offsets [nvox+1], order [n_kept], sorted rows [n_kept, 4] or None).
        Entries of ``self.order`` past n_kept are unspecified."""
        n = int(self.n_kept.item())
        if n < 0:
            raise VoxError(n, "sph_reorder (device status)")
        rows = self.sorted[:n] if self.sorted is not None else None
        return self.voxel_of, self.offsets, self.order[:n], rows


@torch.no_grad()
def spherical(points: torch.Tensor, sph_min: Sequence[float], sph_cell: Sequence[float],
              bins: Sequence[int], *, sorted_rows: bool = True, points_per_thread: int = 0,
              digit_bits: int = 0, sort_tile: int = 0):
    """Spherical binning and voxel-contiguous reorder: (voxel_of [N] i32, -1 when
    not kept; offsets [nvox+1] i32; order [n_kept] i32; the kept rows in that
    order [n_kept, 4] f32, or None). Reads the kept count back (one sync)."""
    _check_points(points)
    s = SphericalSorter(points.shape[0], sph_min, sph_cell, bins, device=points.device,
                        sorted_rows=sorted_rows, points_per_thread=points_per_thread,
                        digit_bits=digit_bits, sort_tile=sort_tile)
    with torch.cuda.device(points.device):
        s.run(points)
        return s.outputs()
