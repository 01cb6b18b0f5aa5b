"""Seeded synthetic point clouds and operator parameters for pillar voxelization.

This module only *draws inputs*. It holds none of the method's arithmetic
(no binning, no hashing, no grouping), so both the CPU oracle side and the
HIP side can take their inputs from it without sharing any computation.
"""
from .configs import CONFIGS, VoxParams, get_config, config_names  # noqa: F401
from .generate import generate, edge_point_names  # noqa: F401
