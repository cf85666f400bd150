"""MI355X ray-driven X-ray transform pair: Siddon forward projection and its matched adjoint.

``project(volume) -> sinogram`` computes, for every detector pixel of every view, the line
integral of the cell-constant volume along the pixel's ray; ``backproject(sinogram) -> volume``
is its exact transpose (diffct pages, "diffct 2.1.0 -> 2.2.1", README "Why diffct", bullet
"Matched operators"). All arithmetic runs in the HIP kernels of ``libmbp.so`` behind the C ABI
in ``include/mbp.h``; this module only marshals arguments. PyTorch provides device memory and
streams.

Shapes follow the tensor order of the pages' problem statement: volumes ``(D, H, W)`` (2-D:
``(H, W)``), sinograms ``(views, rows, cols)`` (2-D: ``(views, cols)``), each with an optional
leading batch. Voxel spacing is per axis in tensor order.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import _capi
from ._capi import MbpError, MbpValueError

__all__ = ["Plan", "project", "backproject", "convert_layout", "stream_copy", "MbpError",
           "MbpValueError", "library_path"]

library_path = _capi.LIB_PATH


def _torch():
    import torch
    return torch


def _as_f64(a, rows: int, rank: int, name: str) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(a, dtype=np.float64)
    if a.shape != (rows, rank):
        raise ValueError(f"trajectory {name} must have shape ({rows}, {rank}), got {a.shape}")
    return a


class Plan:
    """A validated geometry with its per-view frames.

    Parameters
    ----------
    beam: "parallel" | "fan" (2-D) or "cone" | "parallel3d" (3-D).
    volume_shape: ``(H, W)`` or ``(D, H, W)``.
    voxel_spacing: scalar or per axis in tensor order, ``(dy, dx)`` / ``(dz, dy, dx)``.
    trajectory: dict with ``src`` (source, or ray direction for the parallel beams), ``det``
        (detector centre), ``eu`` and, for 3-D beams, ``ev`` (detector axes), each
        ``(views, rank)``.
    detector_shape: ``cols`` (2-D) or ``(rows, cols)``.
    detector_spacing: ``du`` (2-D) or ``(dv, du)``.
    layout: "DHW" (C order) or "WHD" (z fastest, 3-D beams only) for the caller's volumes.
    center: world position of the volume centre.
    """

    def __init__(self, beam: str, volume_shape: Sequence[int], voxel_spacing, trajectory: dict,
                 detector_shape, detector_spacing=1.0, layout: str = "DHW",
                 center: Optional[Sequence[float]] = None):
        lib = _capi.load()
        if beam not in _capi.BEAMS:
            raise ValueError(f"beam must be one of {sorted(_capi.BEAMS)}")
        if layout not in _capi.LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(_capi.LAYOUTS)}")
        cone = beam in _capi.BEAMS_3D        # a 3-D beam: (D, H, W) volume, (rows, cols) detector
        rank = 3 if cone else 2
        shape = tuple(int(s) for s in volume_shape)
        if len(shape) != rank:
            raise ValueError(f"volume_shape must have {rank} entries for beam {beam!r}")
        sp = np.broadcast_to(np.asarray(voxel_spacing, dtype=np.float64), (rank,))
        if cone:
            rows, cols = (int(d) for d in detector_shape)
            dv, du = (float(x) for x in np.broadcast_to(np.asarray(detector_spacing, np.float64), (2,)))
        else:
            cols = int(np.asarray(detector_shape).reshape(-1)[-1])
            rows = 1
            du = float(np.asarray(detector_spacing, dtype=np.float64).reshape(-1)[-1])
            dv = 1.0
        src = np.asarray(trajectory["src"].detach().cpu() if hasattr(trajectory["src"], "detach") else trajectory["src"])
        views = int(src.shape[0])
        self._arrays = [_as_f64(trajectory[k], views, rank, k) for k in ("src", "det", "eu")]
        self._arrays.append(_as_f64(trajectory["ev"], views, 3, "ev") if cone else None)
        g = _capi.Geometry()
        g.beam = _capi.BEAMS[beam]
        g.layout = _capi.LAYOUTS[layout]
        if cone:
            g.D, g.H, g.W = shape
            g.spacing[0], g.spacing[1], g.spacing[2] = sp
        else:
            g.D, (g.H, g.W) = 1, shape
            g.spacing[0], g.spacing[1], g.spacing[2] = 1.0, sp[0], sp[1]
        c = (0.0, 0.0, 0.0) if center is None else tuple(float(x) for x in center) + (0.0,) * (3 - len(center))
        g.center[0], g.center[1], g.center[2] = c[:3]
        g.views, g.rows, g.cols = views, rows, cols
        g.du, g.dv = du, dv
        self._geometry = g
        handle = ctypes.c_void_p()
        ptr = [None if a is None else a.ctypes.data_as(ctypes.c_void_p) for a in self._arrays]
        _capi.check(lib.mbp_plan_create(ctypes.byref(g), ptr[0], ptr[1], ptr[2], ptr[3],
                                        ctypes.byref(handle)), "mbp_plan_create")
        self._handle = handle
        self._lib = lib
        self.beam, self.layout, self.rank = beam, layout, rank
        self.volume_shape = shape
        self.sino_shape = (views, rows, cols) if cone else (views, cols)
        self.views, self.rows, self.cols = views, rows, cols

    # -- lifecycle -----------------------------------------------------------------------
    def close(self) -> None:
        if getattr(self, "_handle", None) is not None and self._handle.value:
            self._lib.mbp_plan_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- introspection -------------------------------------------------------------------
    @property
    def info(self) -> dict:
        inf = _capi.PlanInfo()
        _capi.check(self._lib.mbp_plan_get_info(self._handle, ctypes.byref(inf)), "mbp_plan_get_info")
        return {"path": _capi.PATH_NAMES[inf.path], "column_capable": bool(inf.column_capable),
                "views_per_launch": inf.views_per_launch, "launches": inf.launches,
                "rays": inf.rays, "voxels": inf.voxels, "members_per_pass": inf.members_per_pass,
                "last_adjoint": _capi.ADJOINT_NAMES[inf.last_adjoint],
                "last_adjoint_walk": _capi.PATH_NAMES[inf.last_adjoint_walk] if inf.last_adjoint else None,
                "last_adjoint_views_per_launch": inf.last_adjoint_views_per_launch,
                "last_forward_walk": _capi.PATH_NAMES[inf.last_forward_walk] if inf.last_forward_walk else None,
                "last_forward_members_per_pass": inf.last_forward_members_per_pass,
                "orbit": inf.orbit, "last_adjoint_orbit": inf.last_adjoint_orbit,
                "last_forward_orbit": inf.last_forward_orbit}

    def set_path(self, path: str) -> None:
        _capi.check(self._lib.mbp_plan_set_path(self._handle, _capi.PATHS[path]), "mbp_plan_set_path")

    def set_adjoint(self, kind: str) -> None:
        """Adjoint kernel of the column walk: "gather" (default), "scatter" or "auto"."""
        _capi.check(self._lib.mbp_plan_set_adjoint(self._handle, _capi.ADJOINTS[kind]), "mbp_plan_set_adjoint")

    def set_orbit(self, enable: bool) -> None:
        """Whether the column walk and the gather adjoint may share their geometry over a turn
        symmetry of the views (on by default; info["orbit"] is the symmetry found)."""
        _capi.check(self._lib.mbp_plan_set_orbit(self._handle, 1 if enable else 0), "mbp_plan_set_orbit")

    def set_view_batch(self, views: int) -> None:
        _capi.check(self._lib.mbp_plan_set_view_batch(self._handle, int(views)), "mbp_plan_set_view_batch")

    def workspace_size(self, batch: int = 1) -> int:
        n = ctypes.c_size_t()
        _capi.check(self._lib.mbp_workspace_size(self._handle, int(batch), ctypes.byref(n)), "mbp_workspace_size")
        return int(n.value)

    def set_workspace(self, tensor=None) -> None:
        """Use a caller-owned device tensor as workspace (None: library-owned)."""
        if tensor is None:
            _capi.check(self._lib.mbp_set_workspace(self._handle, None, 0), "mbp_set_workspace")
            self._ws = None
            return
        self._ws = tensor
        _capi.check(self._lib.mbp_set_workspace(self._handle, ctypes.c_void_p(tensor.data_ptr()),
                                                tensor.numel() * tensor.element_size()),
                    "mbp_set_workspace")

    def segment_count(self) -> int:
        torch = _torch()
        n = ctypes.c_int64()
        _capi.check(self._lib.mbp_segment_count(self._handle, ctypes.byref(n),
                                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)),
                    "mbp_segment_count")
        return int(n.value)

    # -- layouts -------------------------------------------------------------------------
    def _volume_strides(self, batch_dims: int):
        if self.rank == 2:
            H, W = self.volume_shape
            inner = (W, 1)
            n = H * W
        else:
            D, H, W = self.volume_shape
            inner = (W * H, W, 1) if self.layout == "DHW" else (1, D, D * H)
            n = D * H * W
        return (n,) * batch_dims + inner, n

    def empty_volume(self, batch: Optional[int] = None, device=None):
        """An uninitialised volume tensor (optionally batched) in the plan's layout."""
        torch = _torch()
        lead = () if batch is None else (int(batch),)
        strides, n = self._volume_strides(len(lead))
        buf = torch.empty(max(n * (lead[0] if lead else 1), 0), dtype=torch.float32, device=device or "cuda")
        return torch.as_strided(buf, lead + self.volume_shape, strides)

    def _check_volume(self, vol):
        torch = _torch()
        if not isinstance(vol, torch.Tensor) or vol.dtype != torch.float32 or not vol.is_cuda:
            raise ValueError("volume must be a float32 tensor on a HIP device")
        nd = len(self.volume_shape)
        if tuple(vol.shape[-nd:]) != self.volume_shape or vol.dim() not in (nd, nd + 1):
            raise ValueError(f"volume must have shape [B,] {self.volume_shape}, got {tuple(vol.shape)}")
        batch = vol.shape[0] if vol.dim() == nd + 1 else None
        strides, _ = self._volume_strides(0 if batch is None else 1)
        if vol.numel() and tuple(vol.stride()) != strides and not (batch == 1 and tuple(vol.stride()[1:]) == strides[1:]):
            raise ValueError(f"volume strides {tuple(vol.stride())} do not match layout {self.layout} {strides}")
        return batch

    def _check_sino(self, sino):
        torch = _torch()
        if not isinstance(sino, torch.Tensor) or sino.dtype != torch.float32 or not sino.is_cuda:
            raise ValueError("sinogram must be a float32 tensor on a HIP device")
        nd = len(self.sino_shape)
        if tuple(sino.shape[-nd:]) != self.sino_shape or sino.dim() not in (nd, nd + 1):
            raise ValueError(f"sinogram must have shape [B,] {self.sino_shape}, got {tuple(sino.shape)}")
        if not sino.is_contiguous():
            raise ValueError("sinogram must be contiguous")
        return sino.shape[0] if sino.dim() == nd + 1 else None

    # -- operators -----------------------------------------------------------------------
    def project(self, volume, out=None):
        """Forward projection; returns (or fills) a float32 sinogram ``[B,] sino_shape``."""
        torch = _torch()
        batch = self._check_volume(volume)
        lead = () if batch is None else (batch,)
        if out is None:
            out = torch.empty(lead + self.sino_shape, dtype=torch.float32, device=volume.device)
        elif self._check_sino(out) != batch or out.device != volume.device:
            raise ValueError("out does not match the volume's batch or device")
        with torch.cuda.device(volume.device):
            stream = torch.cuda.current_stream(volume.device).cuda_stream
            _capi.check(self._lib.mbp_project(self._handle, ctypes.c_void_p(volume.data_ptr()),
                                              1 if batch is None else batch,
                                              ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream)),
                        "mbp_project")
        return out

    def backproject(self, sinogram, out=None, accumulate: bool = False):
        """Matched backprojection; returns (or fills / adds into) a volume in the plan's layout."""
        torch = _torch()
        batch = self._check_sino(sinogram)
        if out is None:
            if accumulate:
                raise ValueError("accumulate needs an output volume")
            out = self.empty_volume(batch, device=sinogram.device)
        elif self._check_volume(out) != batch or out.device != sinogram.device:
            raise ValueError("out does not match the sinogram's batch or device")
        with torch.cuda.device(sinogram.device):
            stream = torch.cuda.current_stream(sinogram.device).cuda_stream
            _capi.check(self._lib.mbp_backproject(self._handle, ctypes.c_void_p(sinogram.data_ptr()),
                                                  1 if batch is None else batch,
                                                  ctypes.c_void_p(out.data_ptr()), int(bool(accumulate)),
                                                  ctypes.c_void_p(stream)),
                        "mbp_backproject")
        return out


    def normal(self, volume, out=None, sinogram=None):
        """Normal operator ``A^T A volume`` in the plan's layout; ``sinogram`` (optional)
        receives ``A volume``. Returns ``out``."""
        torch = _torch()
        batch = self._check_volume(volume)
        lead = () if batch is None else (batch,)
        if sinogram is None:
            sinogram = torch.empty(lead + self.sino_shape, dtype=torch.float32, device=volume.device)
        elif self._check_sino(sinogram) != batch or sinogram.device != volume.device:
            raise ValueError("sinogram does not match the volume's batch or device")
        if out is None:
            out = self.empty_volume(batch, device=volume.device)
        elif self._check_volume(out) != batch or out.device != volume.device:
            raise ValueError("out does not match the volume's batch or device")
        with torch.cuda.device(volume.device):
            stream = torch.cuda.current_stream(volume.device).cuda_stream
            _capi.check(self._lib.mbp_normal(self._handle, ctypes.c_void_p(volume.data_ptr()),
                                             1 if batch is None else batch,
                                             ctypes.c_void_p(sinogram.data_ptr()),
                                             ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream)),
                        "mbp_normal")
        return out

    def cgls_workspace_size(self, batch: Optional[int], iters: int) -> int:
        n = ctypes.c_size_t()
        _capi.check(self._lib.mbp_cgls_workspace_size(self._handle, 1 if batch is None else int(batch),
                                                      int(iters), ctypes.byref(n)),
                    "mbp_cgls_workspace_size")
        return int(n.value)

    def cgls(self, sinogram, iters: int, x0=None, rtol: float = 0.0, workspace=None):
        """CGLS for ``min ||A x - y||`` from ``x0`` (zeros if None), ``iters`` iterations.

        Returns ``(x, residual_norms)``: the iterate in the plan's layout (``x0`` itself is
        updated in place when given) and a numpy array ``[B?, iters + 1]`` of residual norms."""
        torch = _torch()
        batch = self._check_sino(sinogram)
        if x0 is None:
            x = self.empty_volume(batch, device=sinogram.device)
            x.zero_()
        else:
            if self._check_volume(x0) != batch or x0.device != sinogram.device:
                raise ValueError("x0 does not match the sinogram's batch or device")
            x = x0
        nb = 1 if batch is None else batch
        need = self.cgls_workspace_size(nb, iters)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=sinogram.device)
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace needs {need} bytes")
        hist = np.zeros((nb, int(iters) + 1), dtype=np.float64)
        with torch.cuda.device(sinogram.device):
            stream = torch.cuda.current_stream(sinogram.device).cuda_stream
            _capi.check(self._lib.mbp_cgls(self._handle, ctypes.c_void_p(sinogram.data_ptr()), nb,
                                           ctypes.c_void_p(x.data_ptr()), int(iters), float(rtol),
                                           ctypes.c_void_p(workspace.data_ptr()),
                                           workspace.numel() * workspace.element_size(),
                                           hist.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                           ctypes.c_void_p(stream)),
                        "mbp_cgls")
        return x, (hist[0] if batch is None else hist)


def _plan_from(volume_shape, voxel_spacing, trajectory, detector, beam, layout, center):
    shape, spacing = detector
    return Plan(beam, volume_shape, voxel_spacing, trajectory, shape, spacing, layout, center)


def project(volume, voxel_spacing, trajectory: dict, detector, beam: str = "cone",
            layout: str = "DHW", center=None):
    """One-shot ``project(volume[D,H,W], voxel_spacing, trajectory[views], detector)``.

    ``detector`` is ``(detector_shape, detector_spacing)`` as in :class:`Plan`."""
    nd = 3 if beam in _capi.BEAMS_3D else 2
    plan = _plan_from(tuple(volume.shape[-nd:]), voxel_spacing, trajectory, detector, beam, layout, center)
    return plan.project(volume)


def backproject(sinogram, volume_shape, voxel_spacing, trajectory: dict, detector,
                beam: str = "cone", layout: str = "DHW", center=None):
    """One-shot matched backprojection into a new volume of ``volume_shape``."""
    plan = _plan_from(volume_shape, voxel_spacing, trajectory, detector, beam, layout, center)
    return plan.backproject(sinogram)


def convert_layout(volume, to_whd: bool):
    """Copy ``[B,] (D, H, W)`` volumes between C order and the z-fastest layout."""
    torch = _torch()
    lib = _capi.load()
    if volume.dim() not in (3, 4) or volume.dtype != torch.float32 or not volume.is_cuda:
        raise ValueError("volume must be a float32 [B,] (D, H, W) tensor on a HIP device")
    D, H, W = volume.shape[-3:]
    batch = volume.shape[0] if volume.dim() == 4 else 1
    n = D * H * W
    lead = tuple(volume.shape[:-3])
    if to_whd:
        want_in = (W * H, W, 1)
        out_strides = (1, D, D * H)
    else:
        want_in = (1, D, D * H)
        out_strides = (W * H, W, 1)
    if tuple(volume.stride()[-3:]) != want_in:
        raise ValueError("volume strides do not match the source layout")
    buf = torch.empty(n * batch, dtype=torch.float32, device=volume.device)
    out = torch.as_strided(buf, lead + (D, H, W), (n,) * len(lead) + out_strides)
    with torch.cuda.device(volume.device):
        stream = torch.cuda.current_stream(volume.device).cuda_stream
        _capi.check(lib.mbp_convert_layout(ctypes.c_void_p(volume.data_ptr()), batch, D, H, W,
                                           int(bool(to_whd)), ctypes.c_void_p(out.data_ptr()),
                                           ctypes.c_void_p(stream)), "mbp_convert_layout")
    return out


def stream_copy(src, dst) -> None:
    """``dst[:] = src`` for contiguous float32 device tensors of the same size, with the
    library's streaming copy kernel (the bandwidth reference of the measurements)."""
    torch = _torch()
    for t in (src, dst):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("src and dst must be contiguous float32 tensors on a HIP device")
    if src.numel() != dst.numel():
        raise ValueError("src and dst must have the same number of elements")
    lib = _capi.load()
    with torch.cuda.device(src.device):
        stream = torch.cuda.current_stream(src.device).cuda_stream
        _capi.check(lib.mbp_stream_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                        src.numel(), ctypes.c_void_p(stream)), "mbp_stream_copy")
