"""ctypes wrapper of the CPU replay of the GPU walks (``csrc/hostcheck.cpp``).

The replay compiles the same traversal header as the HIP kernels for the host. Tests use it to
prove that every cell a launch configuration visits lies inside the volume before the
configuration runs on a GPU, and to check the walk logic against the oracle on the CPU.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# MBP_SANITIZED=1 (set by tests/run_sanitized.py) selects the ASan/UBSan build
_SANITIZED = os.environ.get("MBP_SANITIZED") == "1"
_LIB = os.path.join(ROOT, "matched_backprojection_amd", "csrc", "_build", "san" if _SANITIZED else "",
                    "libmbp_hostcheck.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            import importlib.util
            spec = importlib.util.spec_from_file_location(
                "mbp_build", os.path.join(ROOT, "matched_backprojection_amd", "csrc", "build.py"))
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            mod.build_hostcheck(sanitize=_SANITIZED)
        lib = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.mbph_project.argtypes = [I, P, I, P, P, P, P, I, I, I, D, D, P, I64, I64, I64, P, P, P, I, I]
        lib.mbph_backproject.argtypes = [I, P, I, P, P, P, P, I, I, I, D, D, P, P, I64, I64, I64, P]
        lib.mbph_check_rays.argtypes = [I, P, I, P, P, P, I, I, I, D, D, P, I64, P]
        lib.mbph_gather.argtypes = [P, I, P, P, P, I, I, I, D, D, P, I, I, P, P, P, I, I]
        lib.mbph_project_chunked.argtypes = [P, I, P, P, P, I, I, I, D, D, P, P, P, I, I]
        lib.mbph_gather_conflicts.argtypes = [P, I, P, P, P, I, I, I, D, D, I, P, P]
        lib.mbph_tilt_band.argtypes = [P, P, P, P, I, I, I, D, D, I, P, P]
        lib.mbph_tilt_gather.argtypes = [P, P, P, P, I, I, I, D, D, P, I, P, P, P]
        lib.mbph_gather_conflicts.restype = I64
        lib.mbph_fast_inside.argtypes = [P, I, P, P, P, I, I, I, D, D, I, I, P, P]
        lib.mbph_fast_inside.restype = I64
        lib.mbph_tilt_band.restype = I64
        lib.mbph_tilt_gather.restype = I64
        lib.mbph_check_rays.restype = I64
        _lib = lib
    return _lib


_BEAMS_3D = ("cone", "parallel3d")


def frames(geom: dict, traj: dict) -> np.ndarray:
    """Per-view (s, c, u, v) in 3-D, as the plan stages them (2-D: rays in the plane z = 0)."""
    views = int(geom["views"])
    f = np.zeros((views, 12), dtype=np.float64)
    rank = 3 if geom["beam"] in _BEAMS_3D else 2
    f[:, 0:rank] = traj["src"]
    f[:, 3:3 + rank] = traj["det"]
    f[:, 6:6 + rank] = traj["eu"]
    if rank == 3:
        f[:, 9:12] = traj["ev"]
    return f


def box(geom: dict):
    shape = tuple(int(s) for s in geom["shape"])
    spacing = tuple(float(s) for s in geom["spacing"])
    if geom["beam"] in _BEAMS_3D:
        n = (shape[2], shape[1], shape[0])
        p = (spacing[2], spacing[1], spacing[0])
    else:
        n = (shape[1], shape[0], 1)
        p = (spacing[1], spacing[0], 1.0)
    c = tuple(geom.get("center", (0.0, 0.0, 0.0))) + (0.0,) * 3
    lo = np.array([c[a] - 0.5 * n[a] * p[a] for a in range(3)])
    return lo, np.array(p, dtype=np.float64), np.array(n, dtype=np.int32)


# the kernels' ray kinds: lines (both parallel beams), fan and cone segments
_BEAM = {"parallel": 0, "fan": 1, "cone": 2, "parallel3d": 0}
_PATH = {"generic": 1, "column": 2}


def _common(geom, traj):
    f = frames(geom, traj)
    lo, p, n = box(geom)
    hi = lo + n * p
    return f, lo, hi, p, n


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def project(path: str, geom: dict, traj: dict, vol: np.ndarray, orbit: int = 1, turn: int = 0):
    """Replay the forward walk on a (D, H, W) / (H, W) float32 volume; orbit 2 or 4 (generic
    walk; turn: the quarter turn's sense): the walks shared over the turn symmetry of the
    views, as the kernel shares them."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    rows = int(geom.get("rows", 1))
    vol = np.ascontiguousarray(vol, dtype=np.float32)
    views, cols = int(geom["views"]), int(geom["cols"])
    sino = np.zeros((views, rows, cols), dtype=np.float32)
    counts = np.zeros((views, rows, cols), dtype=np.int64)
    viol = ctypes.c_longlong(0)
    sx, sy, sz = 1, int(n[0]), int(n[0] * n[1])
    lib.mbph_project(_PATH[path], _ptr(f), _BEAM[geom["beam"]], _ptr(lo), _ptr(hi), _ptr(p),
                     _ptr(n), views, rows, cols, float(geom.get("du", 1.0)), float(geom.get("dv", 1.0)),
                     _ptr(vol), sx, sy, sz, _ptr(sino), _ptr(counts), ctypes.byref(viol),
                     int(orbit), int(turn))
    if geom["beam"] not in _BEAMS_3D:
        sino, counts = sino[:, 0], counts[:, 0]
    return sino, counts, int(viol.value)


def backproject(path: str, geom: dict, traj: dict, sino: np.ndarray):
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    rows = int(geom.get("rows", 1))
    views, cols = int(geom["views"]), int(geom["cols"])
    s = np.ascontiguousarray(sino, dtype=np.float32).reshape(views, rows, cols)
    vol = np.zeros(int(n[0]) * int(n[1]) * int(n[2]), dtype=np.float64)
    viol = ctypes.c_longlong(0)
    sx, sy, sz = 1, int(n[0]), int(n[0] * n[1])
    lib.mbph_backproject(_PATH[path], _ptr(f), _BEAM[geom["beam"]], _ptr(lo), _ptr(hi), _ptr(p),
                         _ptr(n), views, rows, cols, float(geom.get("du", 1.0)),
                         float(geom.get("dv", 1.0)), _ptr(s), _ptr(vol), sx, sy, sz,
                         ctypes.byref(viol))
    return vol.reshape(tuple(int(x) for x in geom["shape"])), int(viol.value)


def check_rays(path: str, geom: dict, traj: dict, ray_ids) -> tuple:
    """Walk selected rays with bounds checks only; returns (visits, violations)."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    ids = np.ascontiguousarray(ray_ids, dtype=np.int64)
    viol = ctypes.c_longlong(0)
    visits = lib.mbph_check_rays(_PATH[path], _ptr(f), _BEAM[geom["beam"]], _ptr(lo), _ptr(p),
                                 _ptr(n), int(geom["views"]), int(geom.get("rows", 1)),
                                 int(geom["cols"]), float(geom.get("du", 1.0)),
                                 float(geom.get("dv", 1.0)), _ptr(ids), ids.size, ctypes.byref(viol))
    return int(visits), int(viol.value)


def gather(geom: dict, traj: dict, sino: np.ndarray, kernel_shares: bool = True,
           general_only: bool = False, orbit: int = 1, turn: int = 0):
    """Replay the cell-gather adjoint item by item (fast fixed-point items with fp32 shares as
    the kernel computes them, or fp64 shares from the same integers; fp64 sums) on a
    (views, rows, cols) sinogram; general_only takes every item in the fp64 general form.
    orbit 2 or 4 (turn: the quarter turn's sense): items shared over the turn symmetry of the
    views, as the kernel forms them. Returns (volume, violations, items in the fast form)."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    rows = int(geom.get("rows", 1))
    views, cols = int(geom["views"]), int(geom["cols"])
    s = np.ascontiguousarray(sino, dtype=np.float32).reshape(views, rows, cols)
    vol = np.zeros(int(n[0]) * int(n[1]) * int(n[2]), dtype=np.float64)
    viol, fast = ctypes.c_longlong(0), ctypes.c_longlong(0)
    lib.mbph_gather(_ptr(f), _BEAM[geom["beam"]], _ptr(lo), _ptr(p), _ptr(n), views, rows, cols,
                    float(geom.get("du", 1.0)), float(geom.get("dv", 1.0)), _ptr(s),
                    int(kernel_shares), int(general_only), _ptr(vol), ctypes.byref(viol),
                    ctypes.byref(fast), int(orbit), int(turn))
    return vol.reshape(tuple(int(x) for x in geom["shape"])), int(viol.value), int(fast.value)


def gather_conflicts(geom: dict, traj: dict, mode: int = 0):
    """(items checked, instructions or steps that fail: lanes that would touch one z cell
    twice, or a combined run that loses, repeats or misdirects a share; fast items checked).
    mode 0: the kernel's grouping; 1 to 4: planted mistakes (see hostcheck.cpp)."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    viol, fast = ctypes.c_longlong(0), ctypes.c_longlong(0)
    checked = lib.mbph_gather_conflicts(_ptr(f), _BEAM[geom["beam"]], _ptr(lo), _ptr(p), _ptr(n),
                                        int(geom["views"]), int(geom.get("rows", 1)),
                                        int(geom["cols"]), float(geom.get("du", 1.0)),
                                        float(geom.get("dv", 1.0)), int(mode), ctypes.byref(viol),
                                        ctypes.byref(fast))
    return int(checked), int(viol.value), int(fast.value)


def fast_inside(geom: dict, traj: dict, zchunk: int, mode: int = 0):
    """(fast items, (item, z chunk) pairs the gather writes without clamping pair indices, rows
    of those whose pair index leaves the chunk's range). mode 1: a planted mistake (the test
    looks at the first row only)."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    inside, viol = ctypes.c_longlong(0), ctypes.c_longlong(0)
    fast = lib.mbph_fast_inside(_ptr(f), _BEAM[geom["beam"]], _ptr(lo), _ptr(p), _ptr(n),
                                int(geom["views"]), int(geom.get("rows", 1)), int(geom["cols"]),
                                float(geom.get("du", 1.0)), float(geom.get("dv", 1.0)),
                                int(zchunk), int(mode), ctypes.byref(inside), ctypes.byref(viol))
    return int(fast), int(inside.value), int(viol.value)


def project_chunked(geom: dict, traj: dict, vol: np.ndarray, orbit: int = 1, turn: int = 0):
    """Replay the forward kernel's chunked column walk on a (D, H, W) float32 volume; orbit 2
    or 4 (turn: the quarter turn's sense): walks shared over the turn symmetry of the views,
    as the kernel shares them."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    rows = int(geom.get("rows", 1))
    views, cols = int(geom["views"]), int(geom["cols"])
    vol = np.ascontiguousarray(vol, dtype=np.float32)
    sino = np.zeros((views, rows, cols), dtype=np.float32)
    viol = ctypes.c_longlong(0)
    lib.mbph_project_chunked(_ptr(f), _BEAM[geom["beam"]], _ptr(lo), _ptr(p), _ptr(n), views, rows,
                             cols, float(geom.get("du", 1.0)), float(geom.get("dv", 1.0)),
                             _ptr(vol), _ptr(sino), ctypes.byref(viol), int(orbit), int(turn))
    return sino, int(viol.value)


def tilt_band(geom: dict, traj: dict, stride: int):
    """(crossings, crossings outside the tilted gather's bands, pixels inside the bands) over
    the xy cells every `stride` cells (see hostcheck.cpp)."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    misses, cand = ctypes.c_longlong(0), ctypes.c_longlong(0)
    hits = lib.mbph_tilt_band(_ptr(f), _ptr(lo), _ptr(p), _ptr(n), int(geom["views"]),
                              int(geom.get("rows", 1)), int(geom["cols"]), float(geom.get("du", 1.0)),
                              float(geom.get("dv", 1.0)), int(stride), ctypes.byref(misses),
                              ctypes.byref(cand))
    return int(hits), int(misses.value), int(cand.value)


def tilt_gather(geom: dict, traj: dict, sino: np.ndarray, mode: int = 0):
    """Replay the gather for detectors whose rows do not run along z on a (views, rows, cols)
    sinogram: (volume (D, H, W) fp64, units, units whose run combine fails, units taking LDS
    atomics); mode 1 plants a mistake (see hostcheck.cpp)."""
    lib = _load()
    f, lo, hi, p, n = _common(geom, traj)
    rows, views, cols = int(geom.get("rows", 1)), int(geom["views"]), int(geom["cols"])
    s = np.ascontiguousarray(sino, dtype=np.float32).reshape(views, rows, cols)
    vol = np.zeros(int(n[0]) * int(n[1]) * int(n[2]), dtype=np.float64)
    conflicts, atomic = ctypes.c_longlong(0), ctypes.c_longlong(0)
    units = lib.mbph_tilt_gather(_ptr(f), _ptr(lo), _ptr(p), _ptr(n), views, rows, cols,
                                 float(geom.get("du", 1.0)), float(geom.get("dv", 1.0)), _ptr(s),
                                 int(mode), _ptr(vol), ctypes.byref(conflicts), ctypes.byref(atomic))
    return (vol.reshape(tuple(int(x) for x in geom["shape"])), int(units), int(conflicts.value),
            int(atomic.value))
