"""O7: the oracle approaches analytic line integrals of ellipses/ellipsoids under refinement.

The line integral of a constant-intensity ellipsoid along a ray is intensity x chord, where
the chord solves a quadratic. Voxelising the ellipsoids at pitch h and running the oracle must
approach the analytic sinogram as h shrinks: the error comes from the staircase boundary only,
so it falls roughly in proportion to h. A wrong convention (detector centring, axis map,
rotation sense, magnification, anisotropic pitch) leaves an O(1) error that does not shrink.
"""

import numpy as np
import pytest

from tests._brute import rays_of
from workloads import circular_cone_trajectory, fan_2d_trajectory, parallel_2d_trajectory
from workloads.phantoms import draw_ellipsoids, voxelise


def _analytic(geom, traj, ellipsoids):
    rays = rays_of(geom, traj)
    S = np.array([r[0] for r in rays])
    Dd = np.array([r[1] for r in rays])
    t0 = np.array([r[2] for r in rays])
    t1 = np.array([r[3] for r in rays])
    out = np.zeros(len(rays))
    for c, axes, R, inten in ellipsoids:
        M = R @ np.diag(1.0 / axes ** 2) @ R.T
        q = S - c
        a = np.einsum("ri,ij,rj->r", Dd, M, Dd)
        b = 2 * np.einsum("ri,ij,rj->r", q, M, Dd)
        cc = np.einsum("ri,ij,rj->r", q, M, q) - 1.0
        disc = b * b - 4 * a * cc
        ok = disc > 0
        sq = np.sqrt(np.where(ok, disc, 0.0))
        r1 = (-b - sq) / (2 * a)
        r2 = (-b + sq) / (2 * a)
        lo = np.maximum(r1, t0)
        hi = np.minimum(r2, t1)
        out += inten * np.where(ok & (hi > lo), hi - lo, 0.0) * np.linalg.norm(Dd, axis=1)
    return out


def _errors(oracle, beam, base_shape, base_spacing, geom_extra, traj, ellipsoids,
            shift=None):
    """Relative L1 error at pitch h, h/2, h/4. ``shift`` moves the oracle's volume box (in
    world units) away from where the phantom was voxelised: a planted convention mistake."""
    errs = []
    for level in range(3):
        f = 2 ** level
        shape = tuple(s * f for s in base_shape)
        spacing = tuple(s / f for s in base_spacing)
        geom = dict(geom_extra, beam=beam, shape=shape, spacing=spacing)
        vol = voxelise(shape, spacing, ellipsoids)
        ref = _analytic(geom, traj, ellipsoids)
        if shift is not None:
            geom["center"] = tuple(shift) + (0.0,) * (3 - len(shift))
        p = oracle.project(geom, traj, vol).ravel()
        errs.append(np.abs(p - ref).sum() / np.abs(ref).sum())
    return errs


def _check(errs):
    assert errs[1] < 0.75 * errs[0] and errs[2] < 0.75 * errs[1], errs
    assert errs[2] < 0.04, errs


def test_parallel_ellipses_converge(oracle):
    shape, spacing = (32, 32), (1.0, 1.0)
    ells = draw_ellipsoids(shape, spacing, 5, (3.0, 10.0), (0.1, 1.0), 1)
    traj = parallel_2d_trajectory(30)
    _check(_errors(oracle, "parallel", shape, spacing,
                   {"views": 30, "rows": 1, "cols": 48, "du": 1.0}, traj, ells))


def test_fan_ellipses_converge_anisotropic(oracle):
    shape, spacing = (24, 40), (1.5, 1.0)
    ells = draw_ellipsoids(shape, spacing, 6, (3.0, 12.0), (0.1, 1.0), 2)
    traj = fan_2d_trajectory(24, 60.0, 110.0)
    _check(_errors(oracle, "fan", shape, spacing,
                   {"views": 24, "rows": 1, "cols": 90, "du": 1.0}, traj, ells))


def test_cone_ellipsoids_converge_anisotropic(oracle):
    shape, spacing = (12, 16, 20), (1.5, 1.0, 0.75)
    ells = draw_ellipsoids(shape, spacing, 4, (2.0, 6.0), (0.1, 1.0), 3)
    traj = circular_cone_trajectory(8, 40.0, 60.0)
    _check(_errors(oracle, "cone", shape, spacing,
                   {"views": 8, "rows": 30, "cols": 28, "du": 1.0, "dv": 1.0}, traj, ells))


def test_planted_offset_does_not_converge(oracle):
    """Negative control: a box displaced by half a coarse voxel keeps an O(1) error."""
    shape, spacing = (24, 40), (1.5, 1.0)
    ells = draw_ellipsoids(shape, spacing, 6, (3.0, 12.0), (0.1, 1.0), 2)
    traj = fan_2d_trajectory(24, 60.0, 110.0)
    errs = _errors(oracle, "fan", shape, spacing,
                   {"views": 24, "rows": 1, "cols": 90, "du": 1.0}, traj, ells, shift=(0.5, 0.0))
    assert errs[2] > 0.5 * errs[0] and errs[2] > 0.05, errs
