"""Voxelised ellipse/ellipsoid phantoms, noise and sinogram-shaped fields (float32).

Draw order per ellipsoid, from ``numpy.random.default_rng(seed)``:
1. centre, one uniform per world axis (x, y[, z]) in ``[-(h - a_max), h - a_max]``, where ``h``
   is the half extent of the volume on that axis and ``a_max`` the top of the semi-axis range
   (0 if negative);
2. semi-axes, one uniform per body axis in ``axis_range``;
3. orientation: 2-D, one angle U[0, pi); 3-D, a unit quaternion from 4 standard normals;
4. intensity U[intensity_range].
Ellipsoids add. After all ellipsoids, an optional background U[0, background) is drawn per
voxel in C order of the tensor shape (as float32).

Voxelisation: a voxel gets an ellipsoid's intensity when its centre lies inside (or on) it.
Voxel centres sit at ``-N*pitch/2 + (i + 0.5)*pitch`` per axis (volume centred on the origin),
with world x <-> W, y <-> H, z <-> D.
"""

from __future__ import annotations

import numpy as np

from .configs import Config


def _quat_to_matrix(q: np.ndarray) -> np.ndarray:
    w, x, y, z = q / np.linalg.norm(q)
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
        [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
        [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)],
    ])


def draw_ellipsoids(shape, spacing, n, axis_range, intensity_range, rng):
    """Return the list of ellipsoid parameters ``(centre_xyz, semi_axes, R, intensity)``.

    ``R`` maps body coordinates to world coordinates (columns are the body axes)."""
    if not isinstance(rng, np.random.Generator):
        rng = np.random.default_rng(rng)
    ndim = len(shape)
    # half extents in world (x, y[, z]) order
    half = [0.5 * shape[ndim - 1 - a] * spacing[ndim - 1 - a] for a in range(ndim)]
    amax = axis_range[1]
    out = []
    for _ in range(n):
        centre = np.array([rng.uniform(-max(h - amax, 0.0), max(h - amax, 0.0)) for h in half])
        axes = rng.uniform(axis_range[0], axis_range[1], size=ndim)
        if ndim == 2:
            phi = rng.uniform(0.0, np.pi)
            R = np.array([[np.cos(phi), -np.sin(phi)], [np.sin(phi), np.cos(phi)]])
        else:
            R = _quat_to_matrix(rng.standard_normal(4))
        intensity = rng.uniform(intensity_range[0], intensity_range[1])
        out.append((centre, axes, R, float(intensity)))
    return out


def _axis_centres(n: int, pitch: float) -> np.ndarray:
    return -0.5 * n * pitch + (np.arange(n, dtype=np.float64) + 0.5) * pitch


def voxelise(shape, spacing, ellipsoids) -> np.ndarray:
    """Sum of ellipsoid indicator functions sampled at voxel centres, as float32 ``shape``."""
    ndim = len(shape)
    vol = np.zeros(shape, dtype=np.float32)
    # world coordinate of voxel centres along x, y[, z]
    coords = [_axis_centres(shape[ndim - 1 - a], spacing[ndim - 1 - a]) for a in range(ndim)]
    for centre, axes, R, intensity in ellipsoids:
        # bounding box of the ellipsoid per world axis: centre +- sqrt(sum_j (R_ij a_j)^2)
        ext = np.sqrt(((R * axes[None, :]) ** 2).sum(axis=1))
        sl = []
        for a in range(ndim):
            c = coords[a]
            lo = np.searchsorted(c, centre[a] - ext[a] - 1e-9, side="left")
            hi = np.searchsorted(c, centre[a] + ext[a] + 1e-9, side="right")
            sl.append((lo, hi))
        if any(hi <= lo for lo, hi in sl):
            continue
        # quadratic form (p - c)^T M (p - c) <= 1 with M = R diag(1/a^2) R^T, evaluated by
        # broadcasting the per-axis offsets (world-axis order x, y[, z])
        M = (R / axes[None, :] ** 2) @ R.T
        offs = []
        for a in range(ndim):
            o = coords[a][sl[a][0]:sl[a][1]] - centre[a]
            shp = [1] * ndim
            shp[a] = o.size
            offs.append(o.reshape(shp))
        q = None
        for a in range(ndim):
            for b in range(a, ndim):
                term = (M[a, a] if a == b else 2.0 * M[a, b]) * (offs[a] * offs[b])
                q = term if q is None else q + term
        inside = q <= 1.0
        # world-axis order -> tensor order (reverse axes)
        inside_t = np.transpose(inside, tuple(range(ndim - 1, -1, -1)))
        tsl = tuple(slice(*sl[ndim - 1 - t]) for t in range(ndim))
        vol[tsl] += np.float32(intensity) * inside_t.astype(np.float32)
    return vol


def ellipsoid_phantom(shape, spacing, n, axis_range=(10.0, 100.0),
                      intensity_range=(0.1, 1.0), seed=0, background=0.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    ells = draw_ellipsoids(shape, spacing, n, axis_range, intensity_range, rng)
    vol = voxelise(shape, spacing, ells)
    if background > 0.0:
        vol += rng.random(shape, dtype=np.float32) * np.float32(background)
    return vol


def config_phantom(cfg: Config) -> np.ndarray:
    """Phantom(s) of a configuration in tensor order: ``shape`` or ``(B, *shape)``."""
    vols = [ellipsoid_phantom(cfg.shape, cfg.spacing, cfg.n_ellipsoids, cfg.axis_range,
                              cfg.intensity_range, seed, cfg.background)
            for seed in cfg.phantom_seeds[:cfg.members]]
    if cfg.batch:
        return np.stack(vols, axis=0)
    return vols[0]


def add_noise(sino: np.ndarray, sigma: float, seed: int) -> np.ndarray:
    """``sino + N(0, sigma^2)`` in float32 (sigma is the standard deviation)."""
    rng = np.random.default_rng(seed)
    noise = rng.standard_normal(sino.shape, dtype=np.float32) * np.float32(sigma)
    return (sino.astype(np.float32) + noise).astype(np.float32)


def sinogram_field(shape, seed: int, bumps: int = 8, sigma: float = 0.01) -> np.ndarray:
    """A smooth, mostly positive sinogram-shaped field plus N(0, sigma^2) noise, float32.

    Stands in for a measured sinogram where computing the true projection of the phantom
    would take the fp64 oracle minutes (the full-size adjoint parity cases): a sum of
    ``bumps`` separable Gaussian bumps over the normalised (view, row, col) index cube.
    Draw order per bump: centre (3 uniforms), widths (3 uniforms in [0.1, 0.5]), amplitude
    U[0.5, 2]; then the noise."""
    rng = np.random.default_rng(seed)
    views, rows, cols = shape[-3:]
    axes = [np.linspace(0.0, 1.0, n, dtype=np.float64) for n in (views, rows, cols)]
    field = np.zeros((views, rows, cols), dtype=np.float32)
    for _ in range(bumps):
        c = rng.uniform(0.0, 1.0, size=3)
        w = rng.uniform(0.1, 0.5, size=3)
        amp = rng.uniform(0.5, 2.0)
        g = [np.exp(-0.5 * ((axes[a] - c[a]) / w[a]) ** 2).astype(np.float32) for a in range(3)]
        field += np.float32(amp) * g[0][:, None, None] * g[1][None, :, None] * g[2][None, None, :]
    lead = shape[:-3]
    if lead:
        field = np.broadcast_to(field, tuple(lead) + field.shape).copy()
        scale = (1.0 + 0.25 * np.arange(int(np.prod(lead)), dtype=np.float32)).reshape(
            tuple(lead) + (1, 1, 1))
        field = field * scale
    noise = rng.standard_normal(field.shape, dtype=np.float32) * np.float32(sigma)
    return (field + noise).astype(np.float32)
