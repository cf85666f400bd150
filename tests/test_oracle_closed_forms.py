"""Pins of the oracle against closed forms, hand cases and exact special cases (no GPU).

O1  chords of a uniform volume with a known value (axis-aligned rays, body diagonals);
O3  a face-aligned sub-box phantom projects to the chord through that sub-box;
O4  2-D parallel beam at 0 and 90 degrees gives exact row and column sums;
O5  parallel sinogram symmetries (90-degree rotation, mirror, half-turn reversal);
O8  a single-voxel phantom lights exactly the pixels whose rays cross the voxel, around the
    central projection of the voxel centre;
O10 3-D parallel beam: horizontal rays with the row axis along z stay inside one z slice and
    reduce to the 2-D parallel transform of that slice; rays along z give column sums;
golden hand-derived cases in tests/golden/hand_cases.json.
"""

import json
import os

import numpy as np
import pytest

from tests._brute import box_chords, ray_arrays
from workloads import (CONFIGS, SMALL_CONFIGS, config_trajectory, parallel_2d_trajectory,
                       parallel_3d_trajectory)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _geom(cfg):
    return {"beam": cfg.beam, "shape": cfg.shape, "spacing": cfg.spacing, "views": cfg.views,
            "rows": cfg.rows, "cols": cfg.cols, "du": cfg.du, "dv": cfg.dv}


def test_golden_hand_cases(oracle):
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 4
    for c in cases:
        traj = {k: np.asarray(v, dtype=np.float64) for k, v in c["traj"].items()}
        traj.setdefault("ev", None)
        vol = np.asarray(c["volume"], dtype=np.float32)
        p = oracle.project(c["geom"], traj, vol)
        assert p.size == 1
        assert abs(float(p.ravel()[0]) - c["value"]) < 1e-12, c["name"]
        cells, lens = oracle.ray_segments(c["geom"], traj, 0, 0, 0)
        assert list(cells) == c["segments"]["cells"], c["name"]
        np.testing.assert_allclose(lens, c["segments"]["lengths"], rtol=0, atol=1e-14)


def test_uniform_volume_chords(oracle):
    # c1: theta = 0 rays run along +x at y = u_j; bins 16..79 cross all 64 columns
    cfg = CONFIGS["c1_parallel2d"]
    p = oracle.project(_geom(cfg), config_trajectory(cfg), np.ones(cfg.shape, np.float32))
    assert np.all(p[0, 16:80] == 64.0)
    assert np.all(p[0, :16] == 0.0) and np.all(p[0, 80:] == 0.0)
    # theta = 90 degrees: same chords along y
    np.testing.assert_allclose(p[45, 16:80], 64.0, rtol=0, atol=1e-12)
    # body diagonal of a 5^3 cube, pitch 0.5: 5 * 0.5 * sqrt(3)
    geom = {"beam": "cone", "shape": (5, 5, 5), "spacing": (0.5, 0.5, 0.5), "views": 2,
            "rows": 1, "cols": 1}
    traj = {"src": np.array([[-3.0, -3.0, -3.0], [3.0, -3.0, 3.0]]),
            "det": np.array([[3.0, 3.0, 3.0], [-3.0, 3.0, -3.0]]),
            "eu": np.array([[1.0, -1.0, 0.0]] * 2), "ev": np.array([[1.0, 1.0, -2.0]] * 2)}
    p = oracle.project(geom, traj, np.ones((5, 5, 5), np.float32))
    np.testing.assert_allclose(p.ravel(), 2.5 * np.sqrt(3.0), rtol=1e-14)
    # square diagonal in 2-D (fan segment corner to corner): 6 * 0.75 * sqrt(2)
    geom = {"beam": "fan", "shape": (6, 6), "spacing": (0.75, 0.75), "views": 1, "rows": 1,
            "cols": 1}
    traj = {"src": np.array([[-5.0, -5.0]]), "det": np.array([[5.0, 5.0]]),
            "eu": np.array([[1.0, -1.0]]), "ev": None}
    p = oracle.project(geom, traj, np.ones((6, 6), np.float32))
    np.testing.assert_allclose(p.ravel(), 4.5 * np.sqrt(2.0), rtol=1e-14)
    # a central fan ray of c2 crosses the full width: 256
    cfg = CONFIGS["c2_fan2d"]
    geom = dict(_geom(cfg), views=1, cols=1)
    traj = {k: (None if v is None else v[:1]) for k, v in config_trajectory(cfg).items()}
    p = oracle.project(geom, traj, np.ones(cfg.shape, np.float32))
    np.testing.assert_allclose(p.ravel(), 256.0, rtol=1e-14)


def test_parallel_row_and_column_sums(oracle):
    """O4 on c1: theta=0 bin j sums row j-16; theta=90 deg bin j sums column 79-j."""
    cfg = CONFIGS["c1_parallel2d"]
    rng = np.random.default_rng(4)
    f = rng.random(cfg.shape).astype(np.float32)
    p = oracle.project(_geom(cfg), config_trajectory(cfg), f)
    f64 = f.astype(np.float64)
    np.testing.assert_allclose(p[0, 16:80], f64.sum(axis=1), rtol=1e-14)
    np.testing.assert_allclose(p[45, 16:80], f64.sum(axis=0)[::-1], rtol=1e-12)
    assert np.all(p[0, :16] == 0) and np.all(p[0, 80:] == 0)
    # anisotropic pitch (dy, dx) = (1, 0.5): row sums scale by dx
    geom = dict(_geom(cfg), spacing=(1.0, 0.5))
    p = oracle.project(geom, config_trajectory(cfg), f)
    np.testing.assert_allclose(p[0, 16:80], 0.5 * f64.sum(axis=1), rtol=1e-14)


def test_parallel_symmetries(oracle):
    """O5: rotate the image +90 deg, mirror it, and reverse the half-turn, on c1's geometry."""
    cfg = CONFIGS["c1_parallel2d"]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(9)
    f = rng.random(cfg.shape).astype(np.float32)
    N = cfg.shape[0]
    # g(x, y) = f(y, -x): g[iy, ix] = f[N-1-ix, iy]   (counter-clockwise rotation by 90 deg)
    iy, ix = np.indices(cfg.shape)
    g = f[N - 1 - ix, iy]
    pf = oracle.project(geom, traj, f)
    pg = oracle.project(geom, traj, g)
    tol = dict(rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(pg[45:], pf[:45], **tol)
    np.testing.assert_allclose(pg[:45], pf[45:, ::-1], **tol)
    # mirror h(x, y) = f(-x, y): P_h(theta, u) = P_f(pi - theta, -u)
    h = f[:, ::-1]
    ph = oracle.project(geom, traj, h)
    np.testing.assert_allclose(ph[1:], pf[:0:-1, ::-1], **tol)
    np.testing.assert_allclose(ph[0], pf[0], **tol)
    # half-turn reversal on [0, 2 pi): p(theta + pi, u) = p(theta, -u)
    full = parallel_2d_trajectory(180)
    th = np.arange(180) * (np.pi / 90)
    full = {"src": np.stack([np.cos(th), np.sin(th)], 1), "det": np.zeros((180, 2)),
            "eu": np.stack([-np.sin(th), np.cos(th)], 1), "ev": None}
    pfull = oracle.project(dict(geom, views=180), full, f)
    np.testing.assert_allclose(pfull[90:], pfull[:90, ::-1], **tol)


def test_sub_box_phantom(oracle):
    """O3: ones on voxels [z0,z1) x [y0,y1) x [x0,x1) project to the chord through that box."""
    cfg = SMALL_CONFIGS["c4_cone512_aniso"]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    D, H, W = cfg.shape
    dz, dy, dx = cfg.spacing
    z0, z1, y0, y1, x0, x1 = 7, 31, 10, 40, 20, 61
    vol = np.zeros(cfg.shape, np.float32)
    vol[z0:z1, y0:y1, x0:x1] = 1.0
    p = oracle.project(geom, traj, vol)
    lo = np.array([-W * dx / 2 + x0 * dx, -H * dy / 2 + y0 * dy, -D * dz / 2 + z0 * dz])
    hi = np.array([-W * dx / 2 + x1 * dx, -H * dy / 2 + y1 * dy, -D * dz / 2 + z1 * dz])
    expect = box_chords(*ray_arrays(geom, traj), lo, hi)
    np.testing.assert_allclose(p.ravel(), expect, rtol=0, atol=1e-10)
    assert (expect > 0).mean() > 0.2


def _detector_coords(src, det, eu, ev, point):
    """(u, v) where the line from src through point meets the detector plane."""
    A = np.stack([eu, ev, -(point - src)], axis=1)
    u, v, _ = np.linalg.solve(A, src - det)
    return u, v


def test_single_voxel_phantom(oracle):
    """O8: exactly the rays that cross the voxel are nonzero; the pixel nearest the central
    projection of the voxel centre is among them and carries a near-maximal chord."""
    cfg = SMALL_CONFIGS["c3_cone256"]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    D, H, W = cfg.shape
    dz, dy, dx = cfg.spacing
    iz, iy, ix = 29, 11, 37
    vol = np.zeros(cfg.shape, np.float32)
    vol[iz, iy, ix] = 1.0
    p = oracle.project(geom, traj, vol)
    lo = np.array([-W * dx / 2 + ix * dx, -H * dy / 2 + iy * dy, -D * dz / 2 + iz * dz])
    hi = lo + np.array([dx, dy, dz])
    expect = box_chords(*ray_arrays(geom, traj), lo, hi).reshape(p.shape)
    np.testing.assert_allclose(p, expect, rtol=0, atol=1e-12)
    centre = 0.5 * (lo + hi)
    for view in range(cfg.views):
        u, v = _detector_coords(traj["src"][view], traj["det"][view], traj["eu"][view],
                                traj["ev"][view], centre)
        j = int(round(u / cfg.du + (cfg.cols - 1) / 2))
        k = int(round(v / cfg.dv + (cfg.rows - 1) / 2))
        assert p[view, k, j] > 0.5 * p[view].max()
        nz = np.argwhere(p[view] > 0)
        assert np.abs(nz[:, 0] - k).max() <= 2 and np.abs(nz[:, 1] - j).max() <= 2


def test_parallel3d_reduces_to_2d_slices(oracle):
    """O10: with ev = z and horizontal ray directions, detector row k at height v_k (mid-slice
    by construction) sees exactly z slice k, so its sinogram row is the 2-D parallel
    projection of that slice with the same angles, columns and pitches. Checked both ways
    (forward and adjoint)."""
    rng = np.random.default_rng(13)
    D, H, W = 6, 10, 12
    spacing = (1.5, 1.0, 0.75)
    x = rng.random((D, H, W)).astype(np.float32)
    views, cols, du = 9, 17, 0.8
    g3 = {"beam": "parallel3d", "shape": (D, H, W), "spacing": spacing, "views": views,
          "rows": D, "cols": cols, "du": du, "dv": spacing[0]}
    g2 = {"beam": "parallel", "shape": (H, W), "spacing": spacing[1:], "views": views,
          "rows": 1, "cols": cols, "du": du}
    t3 = parallel_3d_trajectory(views)
    t2 = parallel_2d_trajectory(views)
    np.testing.assert_array_equal(t3["src"][:, :2], t2["src"])
    p3 = oracle.project(g3, t3, x)
    for k in range(D):
        np.testing.assert_allclose(p3[:, k, :], oracle.project(g2, t2, x[k]), rtol=0, atol=1e-12)
    y = rng.random((views, D, cols)).astype(np.float32)
    b3 = oracle.backproject(g3, t3, y)
    for k in range(D):
        np.testing.assert_allclose(b3[k], oracle.backproject(g2, t2, y[:, k, :]), rtol=0, atol=1e-12)
    assert np.abs(p3).max() > 1.0


def test_parallel3d_axial_rays_give_column_sums(oracle):
    """O10: rays along +z through voxel centres (eu = x, ev = y, pitches equal to the voxel
    pitches) integrate each (y, x) column: P[row iy, col ix] = dz * sum_z x[z, iy, ix]."""
    rng = np.random.default_rng(14)
    D, H, W = 5, 4, 6
    spacing = (1.25, 0.5, 0.75)
    x = rng.random((D, H, W)).astype(np.float32)
    g = {"beam": "parallel3d", "shape": (D, H, W), "spacing": spacing, "views": 1,
         "rows": H, "cols": W, "du": spacing[2], "dv": spacing[1]}
    t = {"src": np.array([[0.0, 0.0, 1.0]]), "det": np.array([[0.0, 0.0, -7.0]]),
         "eu": np.array([[1.0, 0.0, 0.0]]), "ev": np.array([[0.0, 1.0, 0.0]])}
    p = oracle.project(g, t, x)
    np.testing.assert_allclose(p[0], spacing[0] * x.astype(np.float64).sum(axis=0), rtol=1e-14)
