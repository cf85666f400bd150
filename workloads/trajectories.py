"""Per-view trajectory arrays in float64.

Each view carries its own source (or, for parallel beams, ray direction), detector centre and
detector axes, as on the diffct pages (page "diffct 2.2.1 -> 2.4.0", README "Why diffct":
arbitrary per-view trajectories; page "diffct 2.1.0 -> 2.2.1", ``diffct/analytical.py``: the
geometry tuples ``(ray_dir, det_origin, det_u_vec)``, ``(src_pos, det_center, det_u_vec)`` and
``(src_pos, det_center, det_u_vec, det_v_vec)``, each of shape ``(n_views, ndim)``).

The trajectory helper definitions themselves are not on the pages, so the circular and
helical orbits below are the plainest reading: the source turns counter-clockwise about the
z axis, the flat detector faces it through the isocentre at distance SDD from the source,
``det_u`` is the in-plane tangent and ``det_v`` is +z.

Returned dict keys: ``src``, ``det``, ``eu`` and ``ev`` (``ev`` is ``None`` for 2-D beams).
"""

from __future__ import annotations

import numpy as np

from .configs import Config


def parallel_2d_trajectory(views: int) -> dict:
    """2-D parallel beam, angles k*pi/views over [0, pi)."""
    theta = np.arange(views, dtype=np.float64) * (np.pi / views)
    c, s = np.cos(theta), np.sin(theta)
    return {
        "src": np.stack([c, s], axis=1),                 # ray direction
        "det": np.zeros((views, 2), dtype=np.float64),    # detector line through the origin
        "eu": np.stack([-s, c], axis=1),
        "ev": None,
    }


def fan_2d_trajectory(views: int, sid: float, sdd: float) -> dict:
    """2-D fan beam with a flat detector, angles 2*pi*k/views over [0, 2*pi)."""
    theta = np.arange(views, dtype=np.float64) * (2.0 * np.pi / views)
    c, s = np.cos(theta), np.sin(theta)
    return {
        "src": np.stack([sid * c, sid * s], axis=1),
        "det": np.stack([(sid - sdd) * c, (sid - sdd) * s], axis=1),
        "eu": np.stack([-s, c], axis=1),
        "ev": None,
    }


def _cone(theta: np.ndarray, z: np.ndarray, sid: float, sdd: float) -> dict:
    c, s = np.cos(theta), np.sin(theta)
    n = theta.shape[0]
    zero = np.zeros(n, dtype=np.float64)
    one = np.ones(n, dtype=np.float64)
    return {
        "src": np.stack([sid * c, sid * s, z], axis=1),
        "det": np.stack([(sid - sdd) * c, (sid - sdd) * s, z], axis=1),
        "eu": np.stack([-s, c, zero], axis=1),
        "ev": np.stack([zero, zero, one], axis=1),
    }


def circular_cone_trajectory(views: int, sid: float, sdd: float) -> dict:
    """Circular cone beam in the z = 0 plane, angles 2*pi*k/views."""
    theta = np.arange(views, dtype=np.float64) * (2.0 * np.pi / views)
    return _cone(theta, np.zeros(views, dtype=np.float64), sid, sdd)


def helical_cone_trajectory(views: int, turns: int, rise_per_turn: float,
                            sid: float, sdd: float) -> dict:
    """Helical cone beam: ``views`` views over ``turns`` turns; the source and the detector
    rise ``rise_per_turn`` per turn, and the orbit's z range is centred on the volume."""
    if views % turns:
        raise ValueError("views must be a multiple of turns")
    per_turn = views // turns
    k = np.arange(views, dtype=np.float64)
    theta = k * (2.0 * np.pi / per_turn)
    z = rise_per_turn * k / per_turn - 0.5 * rise_per_turn * turns
    return _cone(theta, z, sid, sdd)


def random_cone_trajectory(views: int, seed: int, radius: float = 150.0,
                           sdd: float = 260.0, tilt: float = 0.35) -> dict:
    """General cone trajectory with tilted detectors (det_v not parallel to z).

    Per view (draw order): a source direction from 3 normals (normalised), a detector-u axis
    from 3 normals (orthogonalised against the viewing direction), then one in-plane tilt
    angle U[-tilt, tilt] that rotates (u, v) about the viewing direction.
    """
    rng = np.random.default_rng(seed)
    src = np.empty((views, 3))
    det = np.empty((views, 3))
    eu = np.empty((views, 3))
    ev = np.empty((views, 3))
    for i in range(views):
        w = rng.standard_normal(3)
        w /= np.linalg.norm(w)
        a = rng.standard_normal(3)
        a -= a.dot(w) * w
        a /= np.linalg.norm(a)
        b = np.cross(w, a)
        phi = rng.uniform(-tilt, tilt)
        u = np.cos(phi) * a + np.sin(phi) * b
        v = -np.sin(phi) * a + np.cos(phi) * b
        src[i] = radius * w
        det[i] = (radius - sdd) * w
        eu[i] = u
        ev[i] = v
    return {"src": src, "det": det, "eu": eu, "ev": ev}


# In-plane detector rotation of the tilted circular cone (a calibration-sized tilt).
TILT_DEG = 2.0


def tilted_cone_trajectory(views: int, sid: float, sdd: float, tilt_deg: float = TILT_DEG) -> dict:
    """Circular cone trajectory whose detector axes are rotated in the detector plane by
    tilt_deg about the viewing direction, so the row axis is no longer parallel to z."""
    t = circular_cone_trajectory(views, sid, sdd)
    c, s = np.cos(np.radians(tilt_deg)), np.sin(np.radians(tilt_deg))
    eu, ev = t["eu"].copy(), t["ev"].copy()
    t["eu"] = c * eu + s * ev
    t["ev"] = -s * eu + c * ev
    return t


def parallel_3d_trajectory(views: int, tilt: float = 0.0) -> dict:
    """3-D parallel beam on a circle: view k looks along (cos t, sin t, 0), t = k*pi/views, at
    a detector through the origin with eu = (-sin t, cos t, 0) and ev = z; with tilt != 0 the
    detector axes are rotated by `tilt` radians about the viewing direction (ev no longer
    parallel to z)."""
    theta = np.arange(views, dtype=np.float64) * (np.pi / views)
    c, s = np.cos(theta), np.sin(theta)
    zero = np.zeros(views)
    a = np.stack([-s, c, zero], axis=1)
    b = np.tile([0.0, 0.0, 1.0], (views, 1))
    return {
        "src": np.stack([c, s, zero], axis=1),           # ray direction
        "det": np.zeros((views, 3), dtype=np.float64),
        "eu": np.cos(tilt) * a + np.sin(tilt) * b,
        "ev": -np.sin(tilt) * a + np.cos(tilt) * b,
    }


def random_parallel_3d_trajectory(views: int, seed: int, tilt: float = 0.35,
                                  offset: float = 2.0) -> dict:
    """General 3-D parallel beam: per view (draw order) a ray direction from 3 normals
    (normalised), a detector-u axis from 3 normals (orthogonalised against it), one in-plane
    tilt U[-tilt, tilt] rotating (u, v) about the direction, and a detector centre offset from
    3 normals times `offset`."""
    rng = np.random.default_rng(seed)
    out = {k: np.empty((views, 3)) for k in ("src", "det", "eu", "ev")}
    for i in range(views):
        w = rng.standard_normal(3)
        w /= np.linalg.norm(w)
        a = rng.standard_normal(3)
        a -= a.dot(w) * w
        a /= np.linalg.norm(a)
        b = np.cross(w, a)
        phi = rng.uniform(-tilt, tilt)
        out["src"][i] = w
        out["eu"][i] = np.cos(phi) * a + np.sin(phi) * b
        out["ev"][i] = -np.sin(phi) * a + np.cos(phi) * b
        out["det"][i] = offset * rng.standard_normal(3)
    return out


def config_trajectory(cfg: Config) -> dict:
    if cfg.beam == "parallel":
        return parallel_2d_trajectory(cfg.views)
    if cfg.beam == "parallel3d":
        return parallel_3d_trajectory(cfg.views)
    if cfg.beam == "fan":
        return fan_2d_trajectory(cfg.views, cfg.sid, cfg.sdd)
    if cfg.trajectory == "helical":
        return helical_cone_trajectory(cfg.views, cfg.turns, cfg.rise_per_turn, cfg.sid, cfg.sdd)
    if cfg.trajectory == "circular_tilted":
        return tilted_cone_trajectory(cfg.views, cfg.sid, cfg.sdd)
    return circular_cone_trajectory(cfg.views, cfg.sid, cfg.sdd)
