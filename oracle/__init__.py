"""CPU oracle for pillar / voxel binning (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg use this package. The GPU library never imports, links or calls it, and it
imports nothing from the GPU library.

``voxelize``, ``voxelize_map``, ``downsample``, ``spherical`` and ``bin_points`` wrap the
sequential C definitions in ``voxelize_oracle.c`` (see its comments for the
passages each step follows and the readings taken where the pages are
silent).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "voxelize_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_voxelize.so")
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]

_lib: Optional[ctypes.CDLL] = None


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction).

    The library is written under a temporary name and renamed into place, so
    a process loading it never sees a partly written file."""
    tmp = f"{output}.{os.getpid()}.tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load a compiled oracle (building the default one if it is missing)."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        path = LIBRARY
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.oracle_bin.argtypes = [vp, ctypes.c_int64, vp, vp, vp, vp, vp]
    lib.oracle_bin.restype = ctypes.c_int
    lib.oracle_voxelize.argtypes = [vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int32,
                                    ctypes.c_int32, vp, vp, vp, vp]
    lib.oracle_voxelize.restype = ctypes.c_int
    lib.oracle_voxelize_map.argtypes = [vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int32,
                                        ctypes.c_int32, vp, vp, vp, vp, vp]
    lib.oracle_voxelize_map.restype = ctypes.c_int
    lib.oracle_downsample.argtypes = [vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int32, vp, vp, vp,
                                      vp]
    lib.oracle_downsample.restype = ctypes.c_int
    lib.oracle_spherical.argtypes = [vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_spherical.restype = ctypes.c_int
    if path == LIBRARY:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _param_arrays(range_, cell, grid):
    r = np.ascontiguousarray(np.asarray(range_, dtype=np.float32).reshape(6))
    c = np.ascontiguousarray(np.asarray(cell, dtype=np.float32).reshape(3))
    g = np.ascontiguousarray(np.asarray(grid, dtype=np.int32).reshape(3))
    return r, c, g


def _points(points: np.ndarray) -> np.ndarray:
    p = np.ascontiguousarray(points, dtype=np.float32)
    if p.ndim != 2 or p.shape[1] != 4:
        raise ValueError("points must be [N, 4] float32")
    return p


def bin_points(points: np.ndarray, range_: Sequence[float], cell: Sequence[float],
               grid: Sequence[int], lib: Optional[ctypes.CDLL] = None
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Per-point (valid bool[N], flattened key int64[N], -1 when rejected)."""
    lib = lib or load()
    p = _points(points)
    r, c, g = _param_arrays(range_, cell, grid)
    n = p.shape[0]
    valid = np.zeros(n, dtype=np.int8)
    key = np.zeros(n, dtype=np.int64)
    lib.oracle_bin(_ptr(p), n, _ptr(r), _ptr(c), _ptr(g), _ptr(valid), _ptr(key))
    return valid.astype(bool), key


def voxelize(points: np.ndarray, range_: Sequence[float], cell: Sequence[float],
             grid: Sequence[int], max_points: int, max_voxels: int,
             lib: Optional[ctypes.CDLL] = None
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Return (voxels [V,K,4] f32, coords [V,3] i32 (z,y,x), num_points [V] i32)."""
    lib = lib or load()
    p = _points(points)
    r, c, g = _param_arrays(range_, cell, grid)
    K, M = int(max_points), int(max_voxels)
    if K <= 0 or M <= 0:
        raise ValueError("max_points and max_voxels must be positive")
    # outputs start as all-ones bits so rows the definition leaves unwritten show up
    voxels = np.full((M, K, 4), 0xFFFFFFFF, dtype=np.uint32).view(np.float32)
    coords = np.full((M, 3), -1, dtype=np.int32)
    counts = np.full((M,), -1, dtype=np.int32)
    nv = np.zeros(1, dtype=np.int32)
    rc = lib.oracle_voxelize(_ptr(p), p.shape[0], _ptr(r), _ptr(c), _ptr(g), K, M,
                             _ptr(voxels), _ptr(coords), _ptr(counts), _ptr(nv))
    if rc != 0:
        raise MemoryError("oracle_voxelize could not allocate its dictionary")
    V = int(nv[0])
    return voxels[:V].copy(), coords[:V].copy(), counts[:V].copy()


def voxelize_map(points: np.ndarray, range_: Sequence[float], cell: Sequence[float],
                 grid: Sequence[int], max_points: int, max_voxels: int,
                 lib: Optional[ctypes.CDLL] = None):
    """``voxelize`` plus the inverse map ``point_pillar [N] i32`` (pillar id of
    each point's cell when that pillar is kept, else -1)."""
    lib = lib or load()
    p = _points(points)
    r, c, g = _param_arrays(range_, cell, grid)
    K, M = int(max_points), int(max_voxels)
    if K <= 0 or M <= 0:
        raise ValueError("max_points and max_voxels must be positive")
    voxels = np.full((M, K, 4), 0xFFFFFFFF, dtype=np.uint32).view(np.float32)
    coords = np.full((M, 3), -1, dtype=np.int32)
    counts = np.full((M,), -1, dtype=np.int32)
    pmap = np.full((p.shape[0],), -2, dtype=np.int32)
    nv = np.zeros(1, dtype=np.int32)
    rc = lib.oracle_voxelize_map(_ptr(p), p.shape[0], _ptr(r), _ptr(c), _ptr(g), K, M,
                                 _ptr(voxels), _ptr(coords), _ptr(counts), _ptr(nv), _ptr(pmap))
    if rc != 0:
        raise MemoryError("oracle_voxelize_map could not allocate its dictionary")
    V = int(nv[0])
    return voxels[:V].copy(), coords[:V].copy(), counts[:V].copy(), pmap


def downsample(points: np.ndarray, range_: Sequence[float], cell: Sequence[float],
               grid: Sequence[int], max_voxels: int, lib: Optional[ctypes.CDLL] = None
               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Voxel-grid downsampling: (centroids [V,4] f32 (x, y, z, intensity means),
    coords [V,3] i32 (z,y,x), counts [V] i32 (all points of the voxel))."""
    lib = lib or load()
    p = _points(points)
    r, c, g = _param_arrays(range_, cell, grid)
    M = int(max_voxels)
    if M <= 0:
        raise ValueError("max_voxels must be positive")
    cen = np.full((M, 4), 0xFFFFFFFF, dtype=np.uint32).view(np.float32)
    coords = np.full((M, 3), -1, dtype=np.int32)
    counts = np.full((M,), -1, dtype=np.int32)
    nv = np.zeros(1, dtype=np.int32)
    rc = lib.oracle_downsample(_ptr(p), p.shape[0], _ptr(r), _ptr(c), _ptr(g), M, _ptr(cen),
                               _ptr(coords), _ptr(counts), _ptr(nv))
    if rc != 0:
        raise MemoryError("oracle_downsample could not allocate")
    V = int(nv[0])
    return cen[:V].copy(), coords[:V].copy(), counts[:V].copy()


def spherical(points: np.ndarray, sph_min: Sequence[float], sph_cell: Sequence[float],
              bins: Sequence[int], lib: Optional[ctypes.CDLL] = None):
    """Spherical binning and voxel-contiguous order: (voxel_of [N] i32 (-1 when
    not kept), offsets [nvox+1] i32, order [n_kept] i32)."""
    lib = lib or load()
    p = _points(points)
    mn = np.ascontiguousarray(np.asarray(sph_min, dtype=np.float32).reshape(3))
    ce = np.ascontiguousarray(np.asarray(sph_cell, dtype=np.float32).reshape(3))
    b = np.ascontiguousarray(np.asarray(bins, dtype=np.int32).reshape(3))
    nvox = int(b[0]) * int(b[1]) * int(b[2])
    vof = np.full(p.shape[0], -2, dtype=np.int32)
    off = np.full(nvox + 1, -1, dtype=np.int32)
    order = np.full(max(p.shape[0], 1), -1, dtype=np.int32)
    nk = np.zeros(1, dtype=np.int32)
    rc = lib.oracle_spherical(_ptr(p), p.shape[0], _ptr(mn), _ptr(ce), _ptr(b), _ptr(vof),
                              _ptr(off), _ptr(order), _ptr(nk))
    if rc != 0:
        raise MemoryError("oracle_spherical could not allocate")
    return vof, off, order[:int(nk[0])].copy()


def voxelize_params(points: np.ndarray, params, lib: Optional[ctypes.CDLL] = None):
    """``voxelize`` with a ``workloads.VoxParams``-like object."""
    return voxelize(points, params.range_, params.cell, params.grid, params.max_points,
                    params.max_voxels, lib=lib)
