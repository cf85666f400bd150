"""ctypes wrapper around the fp64 CPU oracle (``oracle/siddon_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the library under test never does, and this module never imports it.

All functions take plain numpy arrays:
- ``geom``: a dict with ``beam`` ("parallel" | "fan" | "cone" | "parallel3d"), ``shape`` (tensor order,
  ``(H, W)`` or ``(D, H, W)``), ``spacing`` (tensor order), optional ``center`` (world x, y, z),
  ``views``, ``rows``, ``cols``, ``du``, ``dv``;
- ``traj``: a dict of float64 arrays ``src``, ``det``, ``eu`` and ``ev`` (``None`` for 2-D),
  each ``(views, rank)``;
- volumes in tensor order, float32, optionally with a leading batch;
- sinograms ``[B?, views, rows, cols]`` (2-D beams: ``[B?, views, cols]``), float32 in, fp64 out.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "siddon_oracle.c")
# MBP_SANITIZED=1 (set by tests/run_sanitized.py) selects the ASan/UBSan build
_SANITIZED = os.environ.get("MBP_SANITIZED") == "1"
_LIB_PATH = os.path.join(_HERE, "_build", "san" if _SANITIZED else "", "liboracle.so")
_BEAMS = {"parallel": 0, "fan": 1, "cone": 2, "parallel3d": 3}
_BEAMS_3D = ("cone", "parallel3d")


class _Geom(ctypes.Structure):
    _fields_ = [
        ("beam", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("D", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
        ("dz", ctypes.c_double), ("dy", ctypes.c_double), ("dx", ctypes.c_double),
        ("cx", ctypes.c_double), ("cy", ctypes.c_double), ("cz", ctypes.c_double),
        ("views", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("du", ctypes.c_double), ("dv", ctypes.c_double),
    ]


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math, no FMA contraction); with
    ``sanitize``, a copy built by clang with AddressSanitizer and UndefinedBehaviorSanitizer
    into ``_build/san/`` (for tests/run_sanitized.py)."""
    path = os.path.join(_HERE, "_build", "san", "liboracle.so") if sanitize else _LIB_PATH
    if force or sanitize or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(path), exist_ok=True)
        tmp = path + ".tmp%d" % os.getpid()
        if sanitize:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fPIC", "-shared",
                   "-fopenmp=libgomp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                   "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                   "-fno-sanitize-recover=all", "-o", tmp, _SRC, "-lm", "-lgomp"]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                   "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, path)
    return path


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(sanitize=_SANITIZED)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        G = ctypes.POINTER(_Geom)
        lib.orc_project.argtypes = [G, P, P, P, P, P, I64, P, P, ctypes.c_int]
        lib.orc_project_rays.argtypes = [G, P, P, P, P, P, I64, P, I64, P, P, ctypes.c_int]
        lib.orc_backproject.argtypes = [G, P, P, P, P, P, I64, P, ctypes.c_int]
        lib.orc_backproject_voxels.argtypes = [G, P, P, P, P, P, I64, P, I64, P, ctypes.c_int]
        lib.orc_ray_segments.argtypes = [G, P, P, P, P, I64, I64, I64, P, P, I64]
        lib.orc_ray_segments.restype = I64
        lib.orc_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().orc_max_threads())


def _geom(geom: dict) -> _Geom:
    beam = geom["beam"]
    shape = tuple(int(s) for s in geom["shape"])
    spacing = tuple(float(s) for s in geom["spacing"])
    if beam in _BEAMS_3D:
        D, H, W = shape
        dz, dy, dx = spacing
    else:
        (H, W), D = shape, 1
        (dy, dx), dz = spacing, 1.0
    c = tuple(geom.get("center", (0.0, 0.0, 0.0)))
    c = c + (0.0,) * (3 - len(c))
    rows = int(geom.get("rows", 1))
    return _Geom(_BEAMS[beam], 0, D, H, W, dz, dy, dx, c[0], c[1], c[2],
                 int(geom["views"]), rows, int(geom["cols"]),
                 float(geom.get("du", 1.0)), float(geom.get("dv", 1.0)))


def _traj(traj: dict, beam: str):
    rank = 3 if beam in _BEAMS_3D else 2
    arrs = []
    for key in ("src", "det", "eu", "ev"):
        a = traj.get(key)
        if a is None:
            if key == "ev" and rank == 2:
                arrs.append(None)
                continue
            raise ValueError(f"trajectory is missing {key}")
        a = np.ascontiguousarray(a, dtype=np.float64)
        if a.ndim != 2 or a.shape[1] != rank:
            raise ValueError(f"trajectory {key} must have shape (views, {rank})")
        arrs.append(a)
    return arrs


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _vol_batch(vol: np.ndarray, ndim: int):
    vol = np.ascontiguousarray(vol, dtype=np.float32)
    if vol.ndim == ndim:
        return vol, 1, False
    if vol.ndim == ndim + 1:
        return vol, vol.shape[0], True
    raise ValueError("volume rank does not match the geometry")


def _sino_shape(g: _Geom, beam: str):
    return (g.views, g.rows, g.cols) if beam in _BEAMS_3D else (g.views, g.cols)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def project(geom: dict, traj: dict, vol: np.ndarray, threads: int = 0, counts: bool = False):
    """Full forward projection in fp64. Returns the sinogram (and per-ray segment counts)."""
    lib = _load()
    g = _geom(geom)
    beam = geom["beam"]
    ndim = 3 if beam in _BEAMS_3D else 2
    vol, B, batched = _vol_batch(vol, ndim)
    src, det, eu, ev = _traj(traj, beam)
    sshape = _sino_shape(g, beam)
    out = np.zeros((B,) + sshape, dtype=np.float64)
    cnt = np.zeros(sshape, dtype=np.int64) if counts else None
    _check(lib.orc_project(ctypes.byref(g), _ptr(src), _ptr(det), _ptr(eu), _ptr(ev), _ptr(vol),
                           B, _ptr(out), _ptr(cnt), int(threads)), "project")
    res = out if batched else out[0]
    return (res, cnt) if counts else res


def project_rays(geom: dict, traj: dict, vol: np.ndarray, ray_ids, threads: int = 0,
                 counts: bool = False):
    """Forward projection of selected rays (flat ids view*rows*cols + row*cols + col)."""
    lib = _load()
    g = _geom(geom)
    beam = geom["beam"]
    ndim = 3 if beam in _BEAMS_3D else 2
    vol, B, batched = _vol_batch(vol, ndim)
    src, det, eu, ev = _traj(traj, beam)
    ids = np.ascontiguousarray(ray_ids, dtype=np.int64)
    out = np.zeros((B, ids.size), dtype=np.float64)
    cnt = np.zeros(ids.size, dtype=np.int64) if counts else None
    _check(lib.orc_project_rays(ctypes.byref(g), _ptr(src), _ptr(det), _ptr(eu), _ptr(ev),
                                _ptr(vol), B, _ptr(ids), ids.size, _ptr(out), _ptr(cnt),
                                int(threads)), "project_rays")
    res = out if batched else out[0]
    return (res, cnt) if counts else res


def _sino_batch(sino: np.ndarray, g: _Geom, beam: str):
    sshape = _sino_shape(g, beam)
    sino = np.ascontiguousarray(sino, dtype=np.float32)
    if sino.shape == sshape:
        return sino, 1, False
    if sino.ndim == len(sshape) + 1 and sino.shape[1:] == sshape:
        return sino, sino.shape[0], True
    raise ValueError(f"sinogram shape {sino.shape} does not match {sshape}")


def backproject(geom: dict, traj: dict, sino: np.ndarray, threads: int = 0):
    """Full adjoint (matched backprojection) in fp64, volume in tensor order."""
    lib = _load()
    g = _geom(geom)
    beam = geom["beam"]
    sino, B, batched = _sino_batch(sino, g, beam)
    src, det, eu, ev = _traj(traj, beam)
    vshape = tuple(int(s) for s in geom["shape"])
    out = np.zeros((B,) + vshape, dtype=np.float64)
    _check(lib.orc_backproject(ctypes.byref(g), _ptr(src), _ptr(det), _ptr(eu), _ptr(ev),
                               _ptr(sino), B, _ptr(out), int(threads)), "backproject")
    return out if batched else out[0]


def backproject_voxels(geom: dict, traj: dict, sino: np.ndarray, vox_ids, threads: int = 0):
    """Adjoint at selected voxels (flat tensor-order ids), from the chord definition."""
    lib = _load()
    g = _geom(geom)
    beam = geom["beam"]
    sino, B, batched = _sino_batch(sino, g, beam)
    src, det, eu, ev = _traj(traj, beam)
    ids = np.ascontiguousarray(vox_ids, dtype=np.int64)
    out = np.zeros((B, ids.size), dtype=np.float64)
    _check(lib.orc_backproject_voxels(ctypes.byref(g), _ptr(src), _ptr(det), _ptr(eu), _ptr(ev),
                                      _ptr(sino), B, _ptr(ids), ids.size, _ptr(out),
                                      int(threads)), "backproject_voxels")
    return out if batched else out[0]


def ray_segments(geom: dict, traj: dict, view: int, row: int, col: int):
    """(cells, lengths) of one ray, cells as flat tensor-order voxel ids."""
    lib = _load()
    g = _geom(geom)
    src, det, eu, ev = _traj(traj, geom["beam"])
    cap = 64
    while True:
        cells = np.zeros(cap, dtype=np.int64)
        lens = np.zeros(cap, dtype=np.float64)
        n = lib.orc_ray_segments(ctypes.byref(g), _ptr(src), _ptr(det), _ptr(eu), _ptr(ev),
                                 int(view), int(row), int(col), _ptr(cells), _ptr(lens), cap)
        if n < 0:
            raise RuntimeError(f"oracle ray_segments failed with status {n}")
        if n <= cap:
            return cells[:n], lens[:n]
        cap = int(n)


def system_matrix(geom: dict, traj: dict) -> np.ndarray:
    """Dense system matrix A [n_rays, n_voxels] from the per-ray segment lists (tiny grids)."""
    shape = tuple(int(s) for s in geom["shape"])
    nvox = int(np.prod(shape))
    rows = int(geom.get("rows", 1))
    A = np.zeros((int(geom["views"]) * rows * int(geom["cols"]), nvox))
    for v in range(int(geom["views"])):
        for k in range(rows):
            for j in range(int(geom["cols"])):
                cells, lens = ray_segments(geom, traj, v, k, j)
                r = (v * rows + k) * int(geom["cols"]) + j
                np.add.at(A[r], cells, lens)
    return A


def geom_from_config(cfg) -> dict:
    """Geometry dict of a :class:`workloads.Config`."""
    return {"beam": cfg.beam, "shape": cfg.shape, "spacing": cfg.spacing, "views": cfg.views,
            "rows": cfg.rows, "cols": cfg.cols, "du": cfg.du, "dv": cfg.dv}


# -- Normal operator and CGLS (fp64) -----------------------------------------------------------
#
# The C oracle reads fp32 volumes and sinograms. An fp64 vector a is passed as two fp32 parts,
# hi = fp32(a) and lo = fp32(a - hi), so a = hi + lo to about 2^-48 relative; by linearity
# A a = A hi + A lo, which keeps the operator products at fp64 accuracy.

def _split(a: np.ndarray):
    a = np.asarray(a, dtype=np.float64)
    hi = a.astype(np.float32)
    lo = (a - hi.astype(np.float64)).astype(np.float32)
    return hi, lo


def project64(geom: dict, traj: dict, vol: np.ndarray, threads: int = 0) -> np.ndarray:
    """A vol for an fp64 volume (optionally batched), fp64 result."""
    hi, lo = _split(vol)
    return project(geom, traj, hi, threads) + project(geom, traj, lo, threads)


def backproject64(geom: dict, traj: dict, sino: np.ndarray, threads: int = 0) -> np.ndarray:
    """A^T sino for an fp64 sinogram (optionally batched), fp64 result."""
    hi, lo = _split(sino)
    return backproject(geom, traj, hi, threads) + backproject(geom, traj, lo, threads)


def normal(geom: dict, traj: dict, vol: np.ndarray, threads: int = 0) -> np.ndarray:
    """The normal operator A^T A vol in fp64."""
    return backproject64(geom, traj, project64(geom, traj, vol, threads), threads)


def cgls(geom: dict, traj: dict, y: np.ndarray, iters: int, x0=None, rtol: float = 0.0,
         threads: int = 0):
    """CGLS for min ||A x - y|| (one unbatched problem), in fp64.

    Conjugate gradients applied to the normal equations A^T A x = A^T y in the form that keeps
    the residual r = y - A x (the "CGLS" variant in A. Bjorck, Numerical Methods for Least
    Squares Problems, SIAM 1996, section 7.4): from x0 (zeros if None),
        r = y - A x,  s = A^T r,  p = s,  gamma = ||s||^2
        per iteration: q = A p,  alpha = gamma / ||q||^2,  x += alpha p,  r -= alpha q,
                       s = A^T r,  beta = ||s||^2 / gamma,  gamma = ||s||^2,  p = s + beta p.
    Once ||r|| <= rtol ||y|| (or A^T r = 0, or ||q|| = 0) the iterate stays as it is. Returns
    (x, norms) with norms[k] = ||r_k|| for k = 0..iters (the recursively updated residual).
    """
    y = np.asarray(y, dtype=np.float64)
    ndim = 3 if geom["beam"] in _BEAMS_3D else 2
    shape = tuple(int(s) for s in geom["shape"])
    if len(shape) != ndim:
        raise ValueError("geometry shape does not match the beam")
    x = np.zeros(shape) if x0 is None else np.array(x0, dtype=np.float64)
    r = y - project64(geom, traj, x, threads)
    y_norm = float(np.linalg.norm(y))
    norms = [float(np.linalg.norm(r))]
    active = norms[0] > rtol * y_norm
    s = backproject64(geom, traj, r, threads)
    gamma = float(np.vdot(s, s))
    if not gamma > 0.0:
        active = False
    p = s.copy()
    for _ in range(int(iters)):
        if active:
            q = project64(geom, traj, p, threads)
            delta = float(np.vdot(q, q))
            if delta > 0.0:
                alpha = gamma / delta
                x += alpha * p
                r -= alpha * q
            else:
                active = False
        norms.append(float(np.linalg.norm(r)))
        if active and not norms[-1] > rtol * y_norm:
            active = False
        if active:
            s = backproject64(geom, traj, r, threads)
            gamma_new = float(np.vdot(s, s))
            beta = gamma_new / gamma
            gamma = gamma_new
            p = s + beta * p
            if not gamma > 0.0:
                active = False
    return x, np.array(norms)
