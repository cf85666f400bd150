"""ctypes declarations of the C ABI in ``include/mbp.h`` (argument marshalling only).

The shared library ``libmbp.so`` is built in-tree by ``matched_backprojection_amd/csrc/build.py``.
There is no fallback: if the library is missing or fails to load, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os

# MBP_SANITIZED=1 selects the copy whose host code is built with ASan and UBSan (for the
# sanitizer run of the CPU tests, tests/run_sanitized.py)
LIB_PATH = (os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "_build", "san", "libmbp.so")
            if os.environ.get("MBP_SANITIZED") == "1"
            else os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmbp.so"))

MBP_OK = 0
MBP_EINVAL = -1
MBP_ENONFINITE = -2
MBP_ECOINCIDENT = -3
MBP_ERANGE = -4
MBP_ETOOLARGE = -5
MBP_EHIP = -6
MBP_ENOMEM = -7

BEAMS = {"parallel": 0, "fan": 1, "cone": 2, "parallel3d": 3}
BEAMS_3D = ("cone", "parallel3d")
LAYOUTS = {"DHW": 0, "WHD": 1}
PATHS = {"auto": 0, "generic": 1, "column": 2}
PATH_NAMES = {v: k for k, v in PATHS.items()}
ADJOINTS = {"auto": 0, "gather": 1, "scatter": 2}
ADJOINT_NAMES = {0: None, 1: "gather", 2: "scatter"}

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = (
    "mbp_plan_create", "mbp_plan_destroy", "mbp_plan_get_info", "mbp_plan_set_path",
    "mbp_plan_set_view_batch", "mbp_plan_set_adjoint", "mbp_plan_set_orbit", "mbp_project", "mbp_backproject", "mbp_segment_count",
    "mbp_workspace_size", "mbp_set_workspace", "mbp_convert_layout", "mbp_normal",
    "mbp_cgls_workspace_size", "mbp_cgls", "mbp_status_string", "mbp_last_error",
    "mbp_abi_version", "mbp_stream_copy", "mbp_backproject_noalloc",
)


class Geometry(ctypes.Structure):
    _fields_ = [
        ("beam", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("D", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
        ("spacing", ctypes.c_double * 3), ("center", ctypes.c_double * 3),
        ("views", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("du", ctypes.c_double), ("dv", ctypes.c_double),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32), ("column_capable", ctypes.c_int32),
        ("views_per_launch", ctypes.c_int64), ("launches", ctypes.c_int64),
        ("rays", ctypes.c_int64), ("voxels", ctypes.c_int64),
        ("members_per_pass", ctypes.c_int64),
        ("last_adjoint", ctypes.c_int32), ("last_adjoint_walk", ctypes.c_int32),
        ("last_adjoint_views_per_launch", ctypes.c_int64),
        ("last_forward_walk", ctypes.c_int32), ("last_forward_members_per_pass", ctypes.c_int32),
        ("orbit", ctypes.c_int32), ("last_adjoint_orbit", ctypes.c_int32),
        ("last_forward_orbit", ctypes.c_int32),
    ]


class MbpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class MbpValueError(MbpError, ValueError):
    pass


_lib = None


def load():
    """Load ``libmbp.so`` (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32, I64 = ctypes.c_int32, ctypes.c_int64
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.mbp_plan_create.argtypes = [ctypes.POINTER(Geometry), P, P, P, P, PP]
    lib.mbp_plan_destroy.argtypes = [P]
    lib.mbp_plan_destroy.restype = None
    lib.mbp_plan_get_info.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.mbp_plan_set_path.argtypes = [P, I32]
    lib.mbp_plan_set_view_batch.argtypes = [P, I64]
    lib.mbp_plan_set_adjoint.argtypes = [P, I32]
    lib.mbp_plan_set_orbit.argtypes = [P, I32]
    lib.mbp_project.argtypes = [P, P, I64, P, P]
    lib.mbp_backproject.argtypes = [P, P, I64, P, I32, P]
    lib.mbp_backproject_noalloc.argtypes = [P, P, I64, P, I32, P]
    lib.mbp_segment_count.argtypes = [P, ctypes.POINTER(I64), P]
    lib.mbp_workspace_size.argtypes = [P, I64, ctypes.POINTER(ctypes.c_size_t)]
    lib.mbp_set_workspace.argtypes = [P, P, ctypes.c_size_t]
    lib.mbp_convert_layout.argtypes = [P, I64, I64, I64, I64, I32, P, P]
    lib.mbp_normal.argtypes = [P, P, I64, P, P, P]
    lib.mbp_cgls_workspace_size.argtypes = [P, I64, I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mbp_cgls.argtypes = [P, P, I64, P, I32, ctypes.c_double, P, ctypes.c_size_t,
                             ctypes.POINTER(ctypes.c_double), P]
    lib.mbp_stream_copy.argtypes = [P, P, I64, P]
    lib.mbp_status_string.argtypes = [ctypes.c_int]
    lib.mbp_status_string.restype = ctypes.c_char_p
    lib.mbp_last_error.argtypes = []
    lib.mbp_last_error.restype = ctypes.c_char_p
    lib.mbp_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int, what: str) -> None:
    if status == MBP_OK:
        return
    lib = load()
    msg = (lib.mbp_last_error() or b"").decode() or lib.mbp_status_string(status).decode()
    text = f"{what}: {msg} (status {status})"
    if status in (MBP_EINVAL, MBP_ENONFINITE, MBP_ECOINCIDENT, MBP_ERANGE, MBP_ETOOLARGE):
        raise MbpValueError(status, text)
    raise MbpError(status, text)
