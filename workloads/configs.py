"""Operator parameters and generator recipes for the five benchmark workloads.

The grid geometry of the pillar workloads (0.16 m cells, a 432 x 496 pillar
grid over x in [0, 69.12), y in [-39.68, 39.68)) is the one the "Voxelize"
page reports for its KITTI frame (Fig. 2 caption). The page's table is sized
at 8 x max_voxels ("A fixed table, sized 8x the voxel budget"); the library
derives that size itself, it is not a parameter here.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple


@dataclass(frozen=True)
class VoxParams:
    """Arguments of one voxelize call (everything except the points)."""
    range_: Tuple[float, float, float, float, float, float]  # x_min,y_min,z_min,x_max,y_max,z_max
    cell: Tuple[float, float, float]                        # vx, vy, vz
    grid: Tuple[int, int, int]                              # gx, gy, gz (gz == 1: pillar mode)
    max_points: int                                         # K
    max_voxels: int                                         # M


@dataclass(frozen=True)
class Config:
    name: str
    description: str
    params: VoxParams
    generator: str          # name of the generator in generate.py
    gen_kwargs: Dict = field(default_factory=dict)
    seed: int = 0


PILLAR_RANGE = (0.0, -39.68, -3.0, 69.12, 39.68, 1.0)
PILLAR_CELL = (0.16, 0.16, 4.0)
PILLAR_GRID = (432, 496, 1)

CONFIGS: Dict[str, Config] = {}


def _add(c: Config) -> None:
    CONFIGS[c.name] = c


_add(Config(
    name="tiny",
    description="4,096 uniform points + 32 hand-placed edge points + a 40-point single-cell "
                "cluster (N = 4,168), 432x496 pillar grid at 0.16 m, K=32, M=12,000",
    params=VoxParams(PILLAR_RANGE, PILLAR_CELL, PILLAR_GRID, 32, 12000),
    generator="tiny", gen_kwargs=dict(n_uniform=4096, cluster=40)))

_add(Config(
    name="kitti_frame",
    description="KITTI-shaped frame, N = 122,880: 90% ground returns (azimuth +-45 deg, "
                "range log-uniform on [2, 80] m, z ~ N(-1.2, 0.6) clipped to [-4, 3]) + 10% "
                "uniform clutter; intensity Beta(2,5); 432x496 grid at 0.16 m, K=32, M=12,000",
    params=VoxParams(PILLAR_RANGE, PILLAR_CELL, PILLAR_GRID, 32, 12000),
    generator="kitti", gen_kwargs=dict(n=122880)))

for _n, _tag in ((25000, "25k"), (65536, "65536"), (130000, "130k")):
    _add(Config(
        name=f"uniform_{_tag}",
        description=f"uniform synthetic cloud, N = {_n:,} over the grid's x/y/z range, "
                    "intensity U[0,1); 432x496 grid at 0.16 m, K=32, M=16,000",
        params=VoxParams(PILLAR_RANGE, PILLAR_CELL, PILLAR_GRID, 32, 16000),
        generator="uniform", gen_kwargs=dict(n=_n)))

_add(Config(
    name="dense_multisweep",
    description="dense multi-sweep, N = 2,097,152: 16 copies of a 131,072-point KITTI-shaped "
                "frame, each jittered by N(0, 0.05 m) in x/y/z; 864x992 grid at 0.08 m, K=32, "
                "M=60,000",
    params=VoxParams(PILLAR_RANGE, (0.08, 0.08, 4.0), (864, 992, 1), 32, 60000),
    generator="multisweep", gen_kwargs=dict(frame_n=131072, sweeps=16, jitter=0.05)))

_add(Config(
    name="voxel3d",
    description="3D voxel variant, N = 1,048,576: range log-uniform on [2, 80] m over azimuth "
                "+-90 deg, kept inside x in [0, 70.4), y in [-40, 40); z ~ U[-3, 1); "
                "0.05x0.05x0.1 m voxels on a 1408x1600x40 grid, K=5, M=40,000",
    params=VoxParams((0.0, -40.0, -3.0, 70.4, 40.0, 1.0), (0.05, 0.05, 0.1), (1408, 1600, 40),
                     5, 40000),
    generator="voxel3d", gen_kwargs=dict(n=1048576)))


def config_names():
    return list(CONFIGS)


def get_config(name: str) -> Config:
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {', '.join(CONFIGS)}")
    return CONFIGS[name]


# ------------------------------------------------- spherical binning workloads --
# The RadiusFPS page measures its sampler on one LiDAR scan of N = 65,536
# points and splits (r, elevation, azimuth) uniformly without giving the bin
# counts. The grid below is a plain choice: r in [0, 80) m in 5 m shells,
# elevation over the whole [-pi/2, pi/2) in 10 degree bands, azimuth over
# [-pi, pi) in 5 degree slices (20,736 voxels). The angle parameters are the
# float32 roundings of these values.

@dataclass(frozen=True)
class SphParams:
    """Arguments of one spherical binning call (everything except the points)."""
    sph_min: Tuple[float, float, float]    # r_min, elevation_min, azimuth_min
    sph_cell: Tuple[float, float, float]   # dr, d_elevation, d_azimuth
    bins: Tuple[int, int, int]             # n_r, n_elevation, n_azimuth


@dataclass(frozen=True)
class SphConfig:
    name: str
    description: str
    params: SphParams
    generator: str
    gen_kwargs: Dict = field(default_factory=dict)
    seed: int = 0


def _deg(d: float) -> float:
    return d * 3.141592653589793 / 180.0


SPH_GRID = SphParams((0.0, -3.141592653589793 / 2, -3.141592653589793),
                     (5.0, _deg(10.0), _deg(5.0)), (16, 18, 72))

SPH_CONFIGS: Dict[str, SphConfig] = {}


def _add_sph(c: SphConfig) -> None:
    SPH_CONFIGS[c.name] = c


_add_sph(SphConfig(
    name="lidar_scan_64k",
    description="one 64-beam 360 degree LiDAR scan, N = 65,536: elevations -24.9 to +2.0 "
                "degrees, ground returns from a sensor 1.73 m up, obstacles at log-uniform "
                "range, unordered",
    params=SPH_GRID, generator="lidar_scan", gen_kwargs=dict(n=65536)))
_add_sph(SphConfig(
    name="lidar_scan_1m",
    description="the same scan recipe at N = 1,048,576 (a dense multi-frame cloud)",
    params=SPH_GRID, generator="lidar_scan", gen_kwargs=dict(n=1048576), seed=1))


def sph_config_names():
    return list(SPH_CONFIGS)


def get_sph_config(name: str) -> SphConfig:
    if name not in SPH_CONFIGS:
        raise KeyError(f"unknown spherical workload {name!r}; known: {', '.join(SPH_CONFIGS)}")
    return SPH_CONFIGS[name]
