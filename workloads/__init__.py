"""Seeded synthetic point clouds and operator parameters (pillar voxelization,
voxel-grid downsampling, spherical binning).

This module only *draws inputs*. It holds none of the method's arithmetic
(no binning, no hashing, no grouping), so both the CPU oracle side and the
HIP side can take their inputs from it without sharing any computation.
"""
from .configs import CONFIGS, VoxParams, get_config, config_names  # noqa: F401
from .configs import (SPH_CONFIGS, SphParams, get_sph_config,  # noqa: F401
                      sph_config_names)
from .generate import generate, edge_point_names  # noqa: F401
