"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package only *generates inputs*: per-view trajectories, voxelised ellipse/ellipsoid
phantoms, noise and sinogram-shaped fields. It contains none of the projector arithmetic
(no ray composition, clipping or traversal), so the oracle and the HIP path can both take
their inputs from here without sharing any of the method.

Random numbers come from ``numpy.random.default_rng(seed)`` (PCG64) with the fixed draw
order written down in :mod:`workloads.phantoms`.
"""

from .configs import CONFIGS, SMALL_CONFIGS, Config, get_config
from .phantoms import ellipsoid_phantom, add_noise, sinogram_field, config_phantom
from .trajectories import (
    parallel_2d_trajectory,
    fan_2d_trajectory,
    circular_cone_trajectory,
    helical_cone_trajectory,
    random_cone_trajectory,
    tilted_cone_trajectory,
    parallel_3d_trajectory,
    random_parallel_3d_trajectory,
    config_trajectory,
)

__all__ = [
    "CONFIGS", "SMALL_CONFIGS", "Config", "get_config",
    "ellipsoid_phantom", "add_noise", "sinogram_field", "config_phantom",
    "parallel_2d_trajectory", "fan_2d_trajectory", "circular_cone_trajectory",
    "helical_cone_trajectory", "random_cone_trajectory",
    "tilted_cone_trajectory", "parallel_3d_trajectory",
    "random_parallel_3d_trajectory", "config_trajectory",
]
