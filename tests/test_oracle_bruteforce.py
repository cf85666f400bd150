"""Pins of the oracle against brute force on tiny grids (no GPU).

O2: the oracle's Siddon system matrix equals the brute-force per-voxel chord matrix.
O6: the oracle adjoint equals A^T y of the brute-force matrix; the adjoint identity holds.
O9: per-ray segment counts equal sum over axes of |exit cell - entry cell| + 1.

Ray families (each view of a 1x1 detector is one arbitrary ray): random segments that start
or end inside the box, axis-parallel rays (some lying exactly in grid planes or on the box
faces), rays between lattice points (simultaneous plane crossings), grazing rays, and
infinite parallel lines.
"""

import numpy as np
import pytest

from tests._brute import dense_matrix, rays_of, voxel_boxes

# Dyadic pitches and centres: every grid plane and box face is exactly representable, so the
# tie cases (rays lying in a plane or on a face) are well defined in floating point.
SHAPE3 = (3, 4, 5)                  # (D, H, W)
SPACING3 = (1.5, 1.0, 0.75)         # (dz, dy, dx)
CENTER3 = (0.375, -0.25, 0.5)       # world (x, y, z)
SHAPE2 = (4, 5)
SPACING2 = (1.0, 0.75)
CENTER2 = (0.375, -0.25)


def _box(shape, spacing, center):
    rank = len(shape)
    n = np.array([shape[rank - 1 - a] for a in range(rank)], dtype=float)
    p = np.array([spacing[rank - 1 - a] for a in range(rank)], dtype=float)
    c = np.array(center[:rank], dtype=float)
    return c - 0.5 * n * p, c + 0.5 * n * p, p


def _single_ray_traj(starts, ends, rank):
    """Trajectory whose view i is the segment starts[i] -> ends[i] on a 1x1 detector."""
    n = len(starts)
    eu = np.zeros((n, rank)); eu[:, 0] = 1.0
    traj = {"src": np.asarray(starts, float), "det": np.asarray(ends, float), "eu": eu, "ev": None}
    if rank == 3:
        ev = np.zeros((n, 3)); ev[:, 1] = 1.0
        traj["ev"] = ev
    return traj


def _segment_rays(rank, shape, spacing, center, seed, n_random=600):
    rng = np.random.default_rng(seed)
    lo, hi, p = _box(shape, spacing, center)
    span = hi - lo
    starts, ends = [], []
    # random segments, endpoints in a box 1.6x the volume (some inside, some outside)
    for _ in range(n_random):
        starts.append(lo - 0.3 * span + 1.6 * span * rng.random(rank))
        ends.append(lo - 0.3 * span + 1.6 * span * rng.random(rank))
    # axis-parallel rays: offsets random, on grid planes, on the low and high faces
    for axis in range(rank):
        for mode in range(4):
            for _ in range(12):
                s = lo + span * rng.random(rank)
                e = s.copy()
                s[axis] = lo[axis] - 1.0
                e[axis] = hi[axis] + 1.0
                other = [b for b in range(rank) if b != axis]
                b = other[rng.integers(len(other))]
                if mode == 1:     # exactly in a grid plane
                    s[b] = e[b] = lo[b] + rng.integers(1, int(round(span[b] / p[b]))) * p[b]
                elif mode == 2:   # on the low face (inside, half-open)
                    s[b] = e[b] = lo[b]
                elif mode == 3:   # on the high face (outside, half-open)
                    s[b] = e[b] = hi[b]
                if rng.random() < 0.5:
                    s, e = e, s
                starts.append(s); ends.append(e)
    # lattice point to lattice point (simultaneous crossings), extended beyond the box
    for _ in range(150):
        na = np.array([round(span[a] / p[a]) for a in range(rank)])
        a0 = lo + rng.integers(0, na + 1) * p
        a1 = lo + rng.integers(0, na + 1) * p
        if np.allclose(a0, a1):
            continue
        d = a1 - a0
        starts.append(a0 - 0.7 * d); ends.append(a1 + 0.4 * d)
    # grazing: along a face with a tiny tilt, and ending exactly on a face
    for _ in range(60):
        s = lo + span * rng.random(rank)
        e = lo + span * rng.random(rank)
        b = rng.integers(rank)
        s[b] = lo[b] - 1e-9
        e[b] = lo[b] + 1e-9
        starts.append(s); ends.append(e)
        s2 = lo - 1.0 + 0.0 * span
        e2 = lo + span * rng.random(rank)
        e2[b] = hi[b]
        starts.append(s2); ends.append(e2)
    # segments entirely inside the box
    for _ in range(60):
        starts.append(lo + span * rng.random(rank)); ends.append(lo + span * rng.random(rank))
    return starts, ends


@pytest.mark.parametrize("rank", [2, 3])
def test_siddon_matrix_equals_brute_force_segments(oracle, rank):
    shape, spacing, center = (SHAPE3, SPACING3, CENTER3) if rank == 3 else (SHAPE2, SPACING2, CENTER2)
    starts, ends = _segment_rays(rank, shape, spacing, center, seed=11 + rank)
    traj = _single_ray_traj(starts, ends, rank)
    geom = {"beam": "cone" if rank == 3 else "fan", "shape": shape, "spacing": spacing,
            "center": center + (0.0,) * (3 - len(center)), "views": len(starts), "rows": 1, "cols": 1}
    A_orc = oracle.system_matrix(geom, traj)
    A_bru = dense_matrix(geom, traj)
    assert A_orc.shape == A_bru.shape
    np.testing.assert_allclose(A_orc, A_bru, rtol=0, atol=1e-12)
    assert ((A_orc > 1e-12) == (A_bru > 1e-12)).all()
    assert (A_bru > 0).sum() > 3000          # the rays really cross the grid


@pytest.mark.parametrize("rank", [2, 3])
def test_parallel_lines_equal_brute_force(oracle, rank):
    shape, spacing, center = (SHAPE3, SPACING3, CENTER3) if rank == 3 else (SHAPE2, SPACING2, CENTER2)
    rng = np.random.default_rng(5)
    lo, hi, p = _box(shape, spacing, center)
    n = 400
    dirs = rng.standard_normal((n, rank))
    dirs[:40, 1:] = 0.0                     # axis-parallel lines
    pts = lo + (hi - lo) * rng.random((n, rank))
    pts[:20, 1] = lo[1] + p[1]              # on a grid plane
    eu = np.zeros((n, rank)); eu[:, 0] = 1.0
    traj = {"src": dirs, "det": pts, "eu": eu, "ev": None}
    if rank == 3:
        traj["ev"] = np.tile([0.0, 1.0, 0.0], (n, 1))
    geom = {"beam": "parallel3d" if rank == 3 else "parallel", "shape": shape, "spacing": spacing,
            "center": center + (0.0,) * (3 - len(center)), "views": n, "rows": 1, "cols": 1}
    A_orc = oracle.system_matrix(geom, traj)
    A_bru = dense_matrix(geom, traj)
    np.testing.assert_allclose(A_orc, A_bru, rtol=0, atol=1e-12)
    assert ((A_orc > 1e-12) == (A_bru > 1e-12)).all()


def test_detector_grid_rays_equal_brute_force(oracle):
    """Full detector grids on a random tilted cone trajectory (pixel composition path)."""
    from workloads import random_cone_trajectory
    traj = random_cone_trajectory(6, seed=3, radius=9.0, sdd=16.0)
    geom = {"beam": "cone", "shape": SHAPE3, "spacing": SPACING3, "center": CENTER3,
            "views": 6, "rows": 5, "cols": 7, "du": 1.3, "dv": 0.9}
    np.testing.assert_allclose(oracle.system_matrix(geom, traj), dense_matrix(geom, traj),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("beam", ["parallel", "fan", "cone", "parallel3d"])
def test_adjoint_equals_transpose_of_brute_force(oracle, beam):
    from workloads import (random_cone_trajectory, fan_2d_trajectory, parallel_2d_trajectory,
                           random_parallel_3d_trajectory)
    if beam == "parallel3d":
        traj = random_parallel_3d_trajectory(5, seed=9, offset=1.0)
        geom = {"beam": "parallel3d", "shape": SHAPE3, "spacing": SPACING3, "center": CENTER3,
                "views": 5, "rows": 4, "cols": 6, "du": 1.1, "dv": 1.4}
    elif beam == "cone":
        traj = random_cone_trajectory(5, seed=8, radius=9.0, sdd=16.0)
        geom = {"beam": "cone", "shape": SHAPE3, "spacing": SPACING3, "center": CENTER3,
                "views": 5, "rows": 4, "cols": 6, "du": 1.1, "dv": 1.4}
    elif beam == "fan":
        traj = fan_2d_trajectory(7, 8.0, 14.0)
        geom = {"beam": "fan", "shape": SHAPE2, "spacing": SPACING2, "center": CENTER2,
                "views": 7, "rows": 1, "cols": 9, "du": 0.8}
    else:
        traj = parallel_2d_trajectory(7)
        geom = {"beam": "parallel", "shape": SHAPE2, "spacing": SPACING2, "center": CENTER2,
                "views": 7, "rows": 1, "cols": 9, "du": 0.6}
    A = dense_matrix(geom, traj)
    rng = np.random.default_rng(2)
    shape = geom["shape"]
    three_d = beam in ("cone", "parallel3d")
    sshape = (geom["views"], geom["rows"], geom["cols"]) if three_d else (geom["views"], geom["cols"])
    y = rng.standard_normal(sshape).astype(np.float32)
    x = rng.standard_normal(shape).astype(np.float32)
    bp = oracle.backproject(geom, traj, y)
    np.testing.assert_allclose(bp.ravel(), A.T @ y.astype(np.float64).ravel(), rtol=0, atol=1e-11)
    fp = oracle.project(geom, traj, x)
    np.testing.assert_allclose(fp.ravel(), A @ x.astype(np.float64).ravel(), rtol=0, atol=1e-11)
    # batched inputs give the per-member results
    xb = np.stack([x, 2 * x, -x])
    fpb = oracle.project(geom, traj, xb)
    np.testing.assert_allclose(fpb, np.stack([fp, 2 * fp, -fp]), rtol=1e-15, atol=1e-12)
    yb = np.stack([y, 2 * y])
    bpb = oracle.backproject(geom, traj, yb)
    np.testing.assert_allclose(bpb, np.stack([bp, 2 * bp]), rtol=1e-15, atol=1e-12)
    # the voxel-by-voxel definition agrees too
    ids = np.arange(int(np.prod(shape)))
    np.testing.assert_allclose(oracle.backproject_voxels(geom, traj, y, ids), bp.ravel(),
                               rtol=0, atol=1e-11)


def _cell_of(point, lo, p, n):
    c = np.floor((point - lo) / p).astype(np.int64)
    return np.clip(c, 0, n - 1)


def test_segment_counts_match_cell_steps(oracle):
    """O9: generic rays visit sum_a |c_exit - c_entry| + 1 cells (no simultaneous crossings)."""
    from workloads import random_cone_trajectory
    traj = random_cone_trajectory(10, seed=21, radius=12.0, sdd=22.0)
    geom = {"beam": "cone", "shape": SHAPE3, "spacing": SPACING3, "center": CENTER3,
            "views": 10, "rows": 6, "cols": 8, "du": 0.9, "dv": 1.2}
    lo, hi, p = _box(SHAPE3, SPACING3, CENTER3)
    n = np.array([SHAPE3[2], SHAPE3[1], SHAPE3[0]])
    ids = np.arange(10 * 6 * 8)
    _, counts = oracle.project_rays(geom, traj, np.ones(SHAPE3, np.float32), ids, counts=True)
    lo_b, hi_b = voxel_boxes(geom)
    checked = 0
    for r, (s, d, t0, t1) in enumerate(rays_of(geom, traj)):
        # entry/exit parameters of the whole box, by slab clipping in the test itself
        with np.errstate(divide="ignore"):
            s1 = (lo - s) / d
            s2 = (hi - s) / d
        a0 = max(t0, np.max(np.minimum(s1, s2)))
        a1 = min(t1, np.min(np.maximum(s1, s2)))
        if not a1 > a0:
            assert counts[r] == 0
            continue
        eps = 1e-9 * (a1 - a0)
        ce = _cell_of(s + (a0 + eps) * d, lo, p, n)
        cx = _cell_of(s + (a1 - eps) * d, lo, p, n)
        assert counts[r] == np.abs(cx - ce).sum() + 1
        checked += 1
    assert checked > 100


@pytest.mark.parametrize("name", ["c3_cone256", "c4_cone512_aniso", "c5_helical_b4"])
def test_voxel_adjoint_matches_scatter_adjoint_on_twins(oracle, name):
    """The adjoint at chosen voxels (the chord definition, which the full-size GPU parity
    tests use as their reference) equals the scatter adjoint at every voxel of the cone
    twins. On these grids a voxel's pixel window (the detector box of its corner projections,
    widened by one pixel) keeps a few dozen of the view's thousands of rays, so a window cut
    too tight, or a corner left out of it, loses chords and fails here; the 3x4x5 grid above
    keeps nearly every pixel and cannot show that."""
    from workloads import SMALL_CONFIGS, config_trajectory
    from oracle.oracle import geom_from_config
    cfg = SMALL_CONFIGS[name]
    geom, traj = geom_from_config(cfg), config_trajectory(cfg)
    y = np.random.default_rng(61).random((cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bp = oracle.backproject(geom, traj, y).ravel()
    bv = oracle.backproject_voxels(geom, traj, y, np.arange(cfg.n_voxels))
    scale = float(np.abs(bp).max())
    assert scale > 0
    err = float(np.abs(bv - bp).max()) / scale
    print(f"{cfg.name}: max |voxel - scatter| / max = {err:.2e}")
    assert err <= 1e-12
