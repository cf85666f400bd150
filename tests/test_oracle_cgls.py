"""Pins of the oracle's fp64 normal operator and CGLS against dense linear algebra (no GPU).

The dense matrix is the brute-force chord matrix of tests/_brute.py (every ray clipped against
every voxel box), written independently of the oracle; the reference solutions come from
numpy.linalg.

S1 the fp64 operator products (fp32 hi/lo split) equal the dense matrix products;
S2 CGLS on small full-column-rank systems reaches numpy.linalg.lstsq's least-squares solution;
S3 the first CGLS step from zero is the exact line search along A^T y;
S4 residual norms never increase and equal ||y - A x_k|| recomputed from the iterate;
S5 started at the least-squares point CGLS stays there, and rtol stops it at the threshold.
"""

import numpy as np
import pytest

from tests._brute import dense_matrix
from workloads import parallel_2d_trajectory, random_cone_trajectory


def _problem(kind):
    if kind == "parallel":
        # 11 views: no view at exactly 90 degrees, where cos(pi/2) = 6e-17 tilts the central
        # ray off the grid plane it lies in (a tie the two definitions round differently)
        geom = {"beam": "parallel", "shape": (4, 5), "spacing": (1.0, 0.75),
                "center": (0.375, -0.25, 0.0), "views": 11, "rows": 1, "cols": 9, "du": 0.6}
        traj = parallel_2d_trajectory(11)
    else:
        geom = {"beam": "cone", "shape": (3, 3, 4), "spacing": (1.5, 1.0, 0.75),
                "center": (0.375, -0.25, 0.5), "views": 9, "rows": 5, "cols": 6,
                "du": 0.9, "dv": 1.1}
        traj = random_cone_trajectory(9, seed=21, radius=9.0, sdd=16.0)
    return geom, traj


def _sino_shape(geom):
    if geom["beam"] == "cone":
        return (geom["views"], geom["rows"], geom["cols"])
    return (geom["views"], geom["cols"])


@pytest.mark.parametrize("kind", ["parallel", "cone"])
def test_fp64_products_equal_dense_matrix(oracle, kind):
    """S1: A x and A^T y for fp64 inputs (not representable in fp32) to fp64 rounding."""
    geom, traj = _problem(kind)
    A = dense_matrix(geom, traj)
    rng = np.random.default_rng(3)
    x = rng.standard_normal(geom["shape"]) * (1 + 1e-9 * rng.standard_normal(geom["shape"]))
    y = rng.standard_normal(_sino_shape(geom)) / 3.0
    np.testing.assert_allclose(oracle.project64(geom, traj, x).ravel(), A @ x.ravel(),
                               rtol=0, atol=1e-12 * np.abs(A @ x.ravel()).max())
    np.testing.assert_allclose(oracle.backproject64(geom, traj, y).ravel(), A.T @ y.ravel(),
                               rtol=0, atol=1e-12 * np.abs(A.T @ y.ravel()).max())
    np.testing.assert_allclose(oracle.normal(geom, traj, x).ravel(), A.T @ (A @ x.ravel()),
                               rtol=0, atol=1e-11 * np.abs(A.T @ (A @ x.ravel())).max())


@pytest.mark.parametrize("kind", ["parallel", "cone"])
def test_cgls_reaches_least_squares_solution(oracle, kind):
    """S2: with full column rank, CGLS reaches the unique least-squares point within n steps
    in exact arithmetic; after n + 10 fp64 steps it agrees with lstsq."""
    geom, traj = _problem(kind)
    A = dense_matrix(geom, traj)
    n = A.shape[1]
    assert np.linalg.matrix_rank(A) == n
    rng = np.random.default_rng(5)
    y = rng.random(_sino_shape(geom)) + 0.1 * rng.standard_normal(_sino_shape(geom))
    x_ls = np.linalg.lstsq(A, y.ravel(), rcond=None)[0]
    x, norms = oracle.cgls(geom, traj, y, n + 10)
    assert np.linalg.norm(x.ravel() - x_ls) <= 1e-8 * np.linalg.norm(x_ls)
    assert abs(norms[-1] - np.linalg.norm(A @ x_ls - y.ravel())) <= 1e-9 * np.linalg.norm(y)


def test_cgls_first_step_is_exact_line_search(oracle):
    """S3: from x0 = 0, x1 = t s with s = A^T y and t = ||s||^2 / ||A s||^2."""
    geom, traj = _problem("cone")
    A = dense_matrix(geom, traj)
    y = np.random.default_rng(6).random(_sino_shape(geom))
    s = A.T @ y.ravel()
    t = (s @ s) / np.linalg.norm(A @ s) ** 2
    x1, norms = oracle.cgls(geom, traj, y, 1)
    np.testing.assert_allclose(x1.ravel(), t * s, rtol=1e-12, atol=1e-14 * np.abs(t * s).max())
    np.testing.assert_allclose(norms, [np.linalg.norm(y), np.linalg.norm(y.ravel() - A @ (t * s))],
                               rtol=1e-12)


@pytest.mark.parametrize("kind", ["parallel", "cone"])
def test_cgls_residuals_decrease_and_match_iterates(oracle, kind):
    """S4: ||y - A x_k|| is non-increasing in k, and the recursive residual equals it."""
    geom, traj = _problem(kind)
    A = dense_matrix(geom, traj)
    y = np.random.default_rng(7).random(_sino_shape(geom))
    prev = None
    for k in range(0, 12, 3):
        x, norms = oracle.cgls(geom, traj, y, k)
        true = np.linalg.norm(y.ravel() - A @ x.ravel())
        assert abs(norms[-1] - true) <= 1e-10 * np.linalg.norm(y)
        assert np.all(np.diff(norms) <= 1e-12 * norms[0])
        if prev is not None:
            np.testing.assert_allclose(norms[:len(prev)], prev, rtol=1e-12)
        prev = norms


def test_cgls_start_at_solution_and_threshold(oracle):
    """S5: x0 = the least-squares point stays put (A^T r = 0 up to rounding); with rtol the
    solve freezes at the first iterate whose residual norm is <= rtol ||y||."""
    geom, traj = _problem("parallel")
    A = dense_matrix(geom, traj)
    y = np.random.default_rng(8).random(_sino_shape(geom))
    x_ls = np.linalg.lstsq(A, y.ravel(), rcond=None)[0].reshape(geom["shape"])
    x, norms = oracle.cgls(geom, traj, y, 5, x0=x_ls)
    assert np.linalg.norm(x - x_ls) <= 1e-9 * np.linalg.norm(x_ls)
    assert np.ptp(norms) <= 1e-9 * norms[0]
    _, full = oracle.cgls(geom, traj, y, 15)
    rtol = float(full[6] / np.linalg.norm(y)) * (1 + 1e-9)
    xr, nr = oracle.cgls(geom, traj, y, 15, rtol=rtol)
    k = int(np.argmax(full <= rtol * np.linalg.norm(y)))
    assert k <= 6
    np.testing.assert_allclose(nr[:k + 1], full[:k + 1], rtol=1e-12)
    assert np.all(nr[k:] == nr[k])
    x_k, _ = oracle.cgls(geom, traj, y, k)
    np.testing.assert_allclose(xr, x_k, rtol=1e-12, atol=1e-15)
