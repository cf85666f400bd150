"""Brute-force reference for tiny grids: the chord of every ray through every voxel's own box.

This is a test helper, written independently of the oracle: it does not merge plane
crossings or locate cells by midpoint; it clips each ray against each voxel box separately
(vectorised over voxels) and so yields the dense system matrix straight from the definition
len(r, v) = |ray r  intersected with  voxel v|.

Conventions follow the shared reading of the diffct pages: world x <-> W, y <-> H, z <-> D;
volume box centred on ``center``; pixel (k, j) at det + u_j*eu + v_k*ev with centred u_j, v_k;
fan/cone rays are segments source -> pixel, parallel rays (2-D and 3-D) are full lines; cells
are half-open.
"""

from __future__ import annotations

import numpy as np


def rays_of(geom: dict, traj: dict):
    """List of (start, direction, tmin, tmax) in world coordinates, ray order view, row, col."""
    beam = geom["beam"]
    rank = 3 if beam in ("cone", "parallel3d") else 2
    rows = int(geom.get("rows", 1))
    cols = int(geom["cols"])
    du = float(geom.get("du", 1.0))
    dv = float(geom.get("dv", 1.0))
    out = []
    for i in range(int(geom["views"])):
        src = np.asarray(traj["src"][i], dtype=np.float64)
        det = np.asarray(traj["det"][i], dtype=np.float64)
        eu = np.asarray(traj["eu"][i], dtype=np.float64)
        ev = None if rank == 2 else np.asarray(traj["ev"][i], dtype=np.float64)
        for k in range(rows):
            v = (k - (rows - 1) / 2.0) * dv
            for j in range(cols):
                u = (j - (cols - 1) / 2.0) * du
                p = det + u * eu + (v * ev if ev is not None else 0.0)
                if beam in ("parallel", "parallel3d"):
                    out.append((p, src.copy(), -np.inf, np.inf))
                else:
                    out.append((src.copy(), p - src, 0.0, 1.0))
    return out


def voxel_boxes(geom: dict):
    """Per-voxel (lo, hi) arrays [nvox, rank] in world axis order, voxel order = tensor C order."""
    beam = geom["beam"]
    shape = tuple(int(s) for s in geom["shape"])
    spacing = tuple(float(s) for s in geom["spacing"])
    rank = len(shape)
    center = np.asarray(geom.get("center", (0.0, 0.0, 0.0))[:rank], dtype=np.float64)
    # world axis a <-> tensor axis rank-1-a
    n = [shape[rank - 1 - a] for a in range(rank)]
    pitch = [spacing[rank - 1 - a] for a in range(rank)]
    lo0 = center - 0.5 * np.asarray(n) * np.asarray(pitch)
    idx = np.indices(shape).reshape(rank, -1)          # tensor-order indices per voxel
    lo = np.empty((idx.shape[1], rank))
    hi = np.empty((idx.shape[1], rank))
    for a in range(rank):
        ia = idx[rank - 1 - a]
        lo[:, a] = lo0[a] + ia * pitch[a]
        hi[:, a] = lo0[a] + (ia + 1) * pitch[a]
    assert beam in ("parallel", "fan", "cone", "parallel3d")
    return lo, hi


def chords(start, d, tmin, tmax, lo, hi):
    """Chord length of one ray through each box (rows of lo/hi), half-open boxes."""
    nb, rank = lo.shape
    a0 = np.full(nb, tmin, dtype=np.float64)
    a1 = np.full(nb, tmax, dtype=np.float64)
    ok = np.ones(nb, dtype=bool)
    for a in range(rank):
        if d[a] != 0.0:
            s1 = (lo[:, a] - start[a]) / d[a]
            s2 = (hi[:, a] - start[a]) / d[a]
            a0 = np.maximum(a0, np.minimum(s1, s2))
            a1 = np.minimum(a1, np.maximum(s1, s2))
        else:
            ok &= (lo[:, a] <= start[a]) & (start[a] < hi[:, a])
    length = np.where(ok & (a1 > a0), a1 - a0, 0.0)
    return length * np.linalg.norm(d)


def dense_matrix(geom: dict, traj: dict) -> np.ndarray:
    lo, hi = voxel_boxes(geom)
    rays = rays_of(geom, traj)
    A = np.zeros((len(rays), lo.shape[0]))
    for r, (s, d, t0, t1) in enumerate(rays):
        A[r] = chords(s, d, t0, t1, lo, hi)
    return A


def ray_arrays(geom: dict, traj: dict):
    """The rays of :func:`rays_of` as stacked arrays (S, D, t0, t1)."""
    rays = rays_of(geom, traj)
    return (np.array([r[0] for r in rays]), np.array([r[1] for r in rays]),
            np.array([r[2] for r in rays]), np.array([r[3] for r in rays]))


def box_chords(S, Dd, t0, t1, lo, hi):
    """Chord of many rays (rows of S, Dd) through one half-open box [lo, hi)."""
    a0 = np.array(t0, dtype=np.float64)
    a1 = np.array(t1, dtype=np.float64)
    ok = np.ones(S.shape[0], dtype=bool)
    for a in range(S.shape[1]):
        nz = Dd[:, a] != 0.0
        with np.errstate(divide="ignore", invalid="ignore"):
            s1 = (lo[a] - S[:, a]) / Dd[:, a]
            s2 = (hi[a] - S[:, a]) / Dd[:, a]
        a0 = np.where(nz, np.maximum(a0, np.minimum(s1, s2)), a0)
        a1 = np.where(nz, np.minimum(a1, np.maximum(s1, s2)), a1)
        ok &= nz | ((lo[a] <= S[:, a]) & (S[:, a] < hi[a]))
    return np.where(ok & (a1 > a0), a1 - a0, 0.0) * np.linalg.norm(Dd, axis=1)
