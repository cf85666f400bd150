"""The synthetic workloads: five full-size configurations and reduced-size twins.

The full-size configurations follow the workload shapes of the diffct pages (page "diffct
2.2.1 -> 2.4.0", README performance table: a 512^3 circular cone beam with flat detector) and
the five parity configurations of this project. The reduced twins keep each configuration's
beam, trajectory family, layout, anisotropy and batch but shrink the grid so the fp64 oracle
finishes in seconds; their detector sizes are chosen so the GPU tiling has ragged tails.

Conventions (shared by every consumer, stated once here):
- volume shape is in tensor order: ``(H, W)`` for 2-D beams, ``(D, H, W)`` for cone beams;
- ``spacing`` is the physical voxel pitch in the same tensor order, ``(dy, dx)`` or
  ``(dz, dy, dx)``;
- world axes map x <-> W (fastest tensor axis), y <-> H, z <-> D; the volume box is centred
  on the world origin;
- the sinogram is ``[views, rows, cols]`` (2-D beams: ``rows == 1``), with an optional
  leading batch;
- ``layout`` names how the GPU side stores the volume: ``"DHW"`` (C order of the tensor shape)
  or ``"WHD"`` (z fastest).
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    beam: str                      # "parallel" | "fan" | "cone" | "parallel3d"
    trajectory: str                # "parallel_half" | "circular" | "circular_tilted" | "helical"
    shape: Tuple[int, ...]         # (H, W) or (D, H, W)
    spacing: Tuple[float, ...]     # tensor order
    views: int
    rows: int                      # 1 for 2-D beams
    cols: int
    du: float = 1.0
    dv: float = 1.0
    sid: float = 0.0               # source-to-isocentre distance (fan/cone)
    sdd: float = 0.0               # source-to-detector distance (fan/cone)
    turns: int = 1                 # helical only
    rise_per_turn: float = 0.0     # helical only: source z advance per turn
    layout: str = "DHW"
    batch: int = 0                 # 0: unbatched; B >= 1: leading batch of B volumes
    n_ellipsoids: int = 5
    axis_range: Tuple[float, float] = (4.0, 20.0)
    intensity_range: Tuple[float, float] = (0.1, 1.0)
    phantom_seeds: Tuple[int, ...] = (1,)
    background: float = 0.0        # U[0, background) i.i.d. per voxel, added after ellipsoids
    noise_sigma: float = 0.0       # std of the Gaussian noise added to the adjoint input
    noise_seed: int = 0
    description: str = ""

    @property
    def ndim(self) -> int:
        return len(self.shape)

    @property
    def n_rays(self) -> int:
        return self.views * self.rows * self.cols

    @property
    def n_voxels(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n

    @property
    def members(self) -> int:
        return max(self.batch, 1)


C1 = Config(
    name="c1_parallel2d", beam="parallel", trajectory="parallel_half",
    shape=(64, 64), spacing=(1.0, 1.0), views=90, rows=1, cols=96,
    n_ellipsoids=5, axis_range=(4.0, 20.0), phantom_seeds=(1,),
    noise_sigma=0.01, noise_seed=101,
    description="2-D parallel beam, 64x64, 90 views over [0, pi), 96 bins pitch 1",
)

C2 = Config(
    name="c2_fan2d", beam="fan", trajectory="circular",
    shape=(256, 256), spacing=(1.0, 1.0), views=360, rows=1, cols=512,
    sid=500.0, sdd=1000.0, n_ellipsoids=10, axis_range=(8.0, 80.0), phantom_seeds=(2,),
    description="2-D fan beam, flat detector, 256x256, SID 500, SDD 1000, 360 views, 512 bins",
)

C3 = Config(
    name="c3_cone256", beam="cone", trajectory="circular",
    shape=(256, 256, 256), spacing=(1.0, 1.0, 1.0), views=360, rows=384, cols=384,
    sid=1000.0, sdd=1500.0, n_ellipsoids=10, axis_range=(10.0, 100.0), phantom_seeds=(3,),
    noise_sigma=0.01, noise_seed=103,
    description="circular cone beam, 256^3, SID 1000, SDD 1500, 360 views, 384x384 detector",
)

C4 = Config(
    name="c4_cone512_aniso", beam="cone", trajectory="circular",
    shape=(512, 512, 512), spacing=(1.5, 1.0, 1.0), views=720, rows=512, cols=768,
    sid=1000.0, sdd=1500.0, layout="WHD", n_ellipsoids=20, axis_range=(10.0, 100.0),
    phantom_seeds=(4,), background=0.05,
    description=("circular cone beam, 512^3 stored (W,H,D)-contiguous, (dz,dy,dx)=(1.5,1,1), "
                 "SID 1000, SDD 1500, 720 views, 768 cols x 512 rows"),
)

C5 = Config(
    name="c5_helical_b4", beam="cone", trajectory="helical",
    shape=(256, 512, 512), spacing=(1.0, 1.0, 1.0), views=1440, rows=64, cols=640,
    sid=600.0, sdd=1100.0, turns=3, rise_per_turn=64.0, batch=4,
    n_ellipsoids=10, axis_range=(10.0, 100.0), phantom_seeds=(51, 52, 53, 54),
    description=("helical cone beam, 512x512x256, SID 600, SDD 1100, 3 turns x 480 views, "
                 "+64 z per turn, 640 cols x 64 rows, batch of 4"),
)

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5)}

# The workload of the pages' own timings (page "diffct 2.2.1 -> 2.4.0", README, multi-GPU
# scaling table; the same shape on "diffct 2.1.0 -> 2.2.1" and "diffct 2.4.3 -> 2.4.4"): a
# 512^3 circular cone beam, 360 views, a 1024 x 768 flat detector at pitch 1.25. The pages
# state neither the source distances nor the phantom: SID 1000 and SDD 1500 are taken, with
# c4's phantom recipe on an isotropic grid (own seed), the volume z-fastest. It is timed for
# context next to the headline, and its sampled parity is checked like the five
# configurations'.
PAGES_CONE512 = Config(
    name="pages_cone512_360v", beam="cone", trajectory="circular",
    shape=(512, 512, 512), spacing=(1.0, 1.0, 1.0), views=360, rows=768, cols=1024,
    du=1.25, dv=1.25, sid=1000.0, sdd=1500.0, layout="WHD", n_ellipsoids=20,
    axis_range=(10.0, 100.0), phantom_seeds=(6,), background=0.05,
    description=("circular cone beam, 512^3 stored (W,H,D)-contiguous, spacing 1, SID 1000, "
                 "SDD 1500 (taken: the pages do not state them), 360 views, 1024 cols x 768 rows, "
                 "pitch 1.25"),
)

CONTEXT_CONFIGS = {PAGES_CONE512.name: PAGES_CONE512}

# Reduced twins: same beam/trajectory/layout/batch, small enough for a full fp64 oracle run.
SMALL_CONFIGS = {
    "c1_parallel2d": C1,
    "c2_fan2d": replace(C2, name="c2s_fan2d", shape=(64, 64), views=90, cols=136,
                        sid=125.0, sdd=250.0, axis_range=(2.0, 20.0)),
    "c3_cone256": replace(C3, name="c3s_cone", shape=(40, 48, 56), views=36, rows=100, cols=90,
                          sid=150.0, sdd=225.0, axis_range=(3.0, 16.0)),
    "c4_cone512_aniso": replace(C4, name="c4s_cone_aniso", shape=(48, 64, 64), views=45,
                                rows=70, cols=100, sid=125.0, sdd=187.5, n_ellipsoids=8,
                                axis_range=(3.0, 20.0)),
    "c5_helical_b4": replace(C5, name="c5s_helical_b4", shape=(24, 64, 64), views=90,
                             rows=10, cols=84, sid=75.0, sdd=137.5, turns=3,
                             rise_per_turn=8.0, n_ellipsoids=4, axis_range=(3.0, 12.0)),
}


def get_config(name: str, small: bool = False) -> Config:
    """Look a configuration up by name; ``small=True`` gives its reduced twin."""
    if name in CONFIGS:
        return SMALL_CONFIGS[name] if small else CONFIGS[name]
    for c in SMALL_CONFIGS.values():
        if c.name == name:
            return c
    raise KeyError(name)
