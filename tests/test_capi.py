"""The C ABI on the CPU: symbols, validation, plans and batch-0 calls (no device work).

Every check here runs in the host code of ``libmbp.so`` before any HIP call, so it needs no
GPU: validation happens at plan creation, and plan creation stages nothing.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from matched_backprojection_amd import _capi
from workloads import CONFIGS, SMALL_CONFIGS, config_trajectory, random_cone_trajectory

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _capi.load()


def rows_padded(rows):
    """Rows of the gather's reordered sinogram: zero-padded to whole groups of S * 64 rows,
    S = min(8, ceil(rows / 64))."""
    g = 64 * min(8, -(-rows // 64))
    return -(-rows // g) * g


def gather_sino_floats(cfg):
    """Floats per member of the reordered sinogram: every padded line, plus a tail of eight
    rows that fixed-width row loads may reach past the last line."""
    return cfg.views * cfg.cols * rows_padded(cfg.rows) + 8


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "mbp.h")).read()
    return sorted(set(re.findall(r"\b(mbp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    declared = _declared_symbols()
    assert len(declared) >= 14
    assert set(declared) == set(_capi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.mbp_abi_version() == 4
    assert lib.mbp_status_string(_capi.MBP_ERANGE) == b"geometry out of range"


def _geometry(cfg, layout=None):
    g = _capi.Geometry()
    g.beam = _capi.BEAMS[cfg.beam]
    g.layout = _capi.LAYOUTS[layout or cfg.layout]
    if cfg.beam in _capi.BEAMS_3D:
        g.D, g.H, g.W = cfg.shape
        g.spacing[0], g.spacing[1], g.spacing[2] = cfg.spacing
    else:
        g.D, (g.H, g.W) = 1, cfg.shape
        g.spacing[0], g.spacing[1], g.spacing[2] = 1.0, cfg.spacing[0], cfg.spacing[1]
    g.views, g.rows, g.cols = cfg.views, cfg.rows, cfg.cols
    g.du, g.dv = cfg.du, cfg.dv
    return g


def _create(lib, g, traj):
    arrs = [np.ascontiguousarray(traj[k], dtype=np.float64) if traj.get(k) is not None else None
            for k in ("src", "det", "eu", "ev")]
    ptrs = [None if a is None else a.ctypes.data_as(ctypes.c_void_p) for a in arrs]
    h = ctypes.c_void_p()
    rc = lib.mbp_plan_create(ctypes.byref(g), *ptrs, ctypes.byref(h))
    return rc, h


def _info(lib, h):
    inf = _capi.PlanInfo()
    assert lib.mbp_plan_get_info(h, ctypes.byref(inf)) == 0
    return inf


@pytest.mark.parametrize("name", list(CONFIGS))
def test_configs_plan_and_pick_walks(lib, name):
    cfg = CONFIGS[name]
    rc, h = _create(lib, _geometry(cfg), config_trajectory(cfg))
    assert rc == 0, lib.mbp_last_error()
    inf = _info(lib, h)
    assert inf.rays == cfg.n_rays and inf.voxels == cfg.n_voxels
    if cfg.beam == "cone":
        assert inf.column_capable == 1 and inf.path == 2
    else:
        assert inf.column_capable == 0 and inf.path == 1
    assert inf.views_per_launch == cfg.views and inf.launches == 1
    ws = ctypes.c_size_t()
    assert lib.mbp_workspace_size(h, cfg.members, ctypes.byref(ws)) == 0
    if cfg.beam != "cone":
        assert ws.value == 0
    else:   # z-fastest volume copy (unless used in place) + reordered sinogram for the gather
        nb = min(4, cfg.members)
        direct = cfg.layout == "WHD" and cfg.members == 1
        sino = gather_sino_floats(cfg)
        assert ws.value == 4 * nb * ((0 if direct else cfg.n_voxels) + sino)
    # nothing has been backprojected yet
    assert inf.last_adjoint == 0 and inf.last_adjoint_walk == 0 and inf.last_adjoint_views_per_launch == 0
    assert inf.last_forward_walk == 0 and inf.last_forward_members_per_pass == 0
    # view batching: a ragged split into launches of 7 views; the gather's reordered sinogram
    # then covers the views of one launch
    assert lib.mbp_plan_set_view_batch(h, 7) == 0
    inf = _info(lib, h)
    assert inf.views_per_launch == 7 and inf.launches == -(-cfg.views // 7)
    assert lib.mbp_workspace_size(h, cfg.members, ctypes.byref(ws)) == 0
    if cfg.beam == "cone":
        assert ws.value == 4 * nb * ((0 if direct else cfg.n_voxels) + 7 * cfg.cols * rows_padded(cfg.rows) + 8)
    assert lib.mbp_plan_set_view_batch(h, -1) == _capi.MBP_EINVAL
    # forcing walks
    assert lib.mbp_plan_set_path(h, 1) == 0 and _info(lib, h).path == 1
    want = 0 if cfg.beam == "cone" else _capi.MBP_EINVAL
    assert lib.mbp_plan_set_path(h, 2) == want
    assert lib.mbp_plan_set_path(h, 7) == _capi.MBP_EINVAL
    lib.mbp_plan_destroy(h)


def test_tilted_detector_uses_generic_walk(lib):
    """Random tilted frames, and a circular orbit whose detector is rotated by a few degrees
    in its plane: the row axis is not along z, so the forward takes the generic walk. The
    adjoint's gather (the default) needs a workspace of the volume copy and the reordered
    sinogram, as the column gather does; the scatter adjoint (the generic walk's atomics), or
    a forced generic walk, needs none."""
    from dataclasses import replace
    cfg = SMALL_CONFIGS["c3_cone256"]
    tilted = replace(cfg, trajectory="circular_tilted")
    for traj in (random_cone_trajectory(cfg.views, seed=1, radius=200.0, sdd=350.0),
                 config_trajectory(tilted)):
        rc, h = _create(lib, _geometry(cfg), traj)
        assert rc == 0
        inf = _info(lib, h)
        assert inf.column_capable == 0 and inf.path == 1
        ws = ctypes.c_size_t()
        assert lib.mbp_workspace_size(h, 3, ctypes.byref(ws)) == 0
        assert ws.value == 4 * 2 * (cfg.n_voxels + gather_sino_floats(cfg))
        assert lib.mbp_plan_set_adjoint(h, 2) == 0
        assert lib.mbp_workspace_size(h, 3, ctypes.byref(ws)) == 0 and ws.value == 0
        assert lib.mbp_plan_set_adjoint(h, 0) == 0 and lib.mbp_plan_set_path(h, 1) == 0
        assert lib.mbp_workspace_size(h, 3, ctypes.byref(ws)) == 0 and ws.value == 0
        lib.mbp_plan_destroy(h)


def test_batch_zero_and_bad_calls_do_no_device_work(lib):
    cfg = SMALL_CONFIGS["c3_cone256"]
    rc, h = _create(lib, _geometry(cfg), config_trajectory(cfg))
    assert rc == 0
    # batch 0: nothing to do, NULL buffers allowed, no HIP call made
    assert lib.mbp_project(h, None, 0, None, None) == 0
    assert lib.mbp_backproject(h, None, 0, None, 0, None) == 0
    assert lib.mbp_convert_layout(None, 0, 4, 5, 6, 1, None, None) == 0
    # invalid arguments are rejected before any device work
    assert lib.mbp_project(h, None, -1, None, None) == _capi.MBP_EINVAL
    assert lib.mbp_project(h, None, 1, None, None) == _capi.MBP_EINVAL
    assert lib.mbp_project(None, None, 1, None, None) == _capi.MBP_EINVAL
    assert lib.mbp_backproject(h, ctypes.c_void_p(16), 1, ctypes.c_void_p(32), 2, None) == _capi.MBP_EINVAL
    assert lib.mbp_project(h, ctypes.c_void_p(18), 1, ctypes.c_void_p(32), None) == _capi.MBP_EINVAL
    assert b"aligned" in lib.mbp_last_error()
    assert lib.mbp_convert_layout(ctypes.c_void_p(64), 2, 4, 5, 6, 1, ctypes.c_void_p(64 + 4 * 100), None) == _capi.MBP_EINVAL
    assert b"overlap" in lib.mbp_last_error()
    assert lib.mbp_set_workspace(h, ctypes.c_void_p(8), 64) == _capi.MBP_EINVAL
    assert lib.mbp_set_workspace(h, None, 64) == _capi.MBP_EINVAL
    assert lib.mbp_set_workspace(h, None, 0) == 0
    lib.mbp_plan_destroy(h)
    lib.mbp_plan_destroy(None)
    # the no-allocation backprojection: argument checks as mbp_backproject's; a call whose
    # least need exceeds the library's scratch (four 256 x 512 x 512 members in (D, H, W)
    # order need a z-fastest volume of 256 MiB for even one member) is refused before any
    # device work
    c5 = CONFIGS["c5_helical_b4"]
    rc, h5 = _create(lib, _geometry(c5), config_trajectory(c5))
    assert rc == 0
    assert lib.mbp_backproject_noalloc(h5, None, 0, None, 0, None) == 0
    assert lib.mbp_backproject_noalloc(h5, None, 1, None, 0, None) == _capi.MBP_EINVAL
    assert lib.mbp_backproject_noalloc(h5, ctypes.c_void_p(64), 4, ctypes.c_void_p(128), 2, None) == _capi.MBP_EINVAL
    assert lib.mbp_backproject_noalloc(h5, ctypes.c_void_p(64), 4, ctypes.c_void_p(128), 0, None) == _capi.MBP_ETOOLARGE
    assert b"scratch" in lib.mbp_last_error()
    lib.mbp_plan_destroy(h5)
    # the streaming copy: nothing to do for n = 0, bad arguments rejected before any launch
    assert lib.mbp_stream_copy(None, None, 0, None) == 0
    assert lib.mbp_stream_copy(None, ctypes.c_void_p(64), 4, None) == _capi.MBP_EINVAL
    assert lib.mbp_stream_copy(ctypes.c_void_p(64), ctypes.c_void_p(128), -1, None) == _capi.MBP_EINVAL
    assert lib.mbp_stream_copy(ctypes.c_void_p(68), ctypes.c_void_p(256), 4, None) == _capi.MBP_EINVAL
    assert b"aligned" in lib.mbp_last_error()
    assert lib.mbp_stream_copy(ctypes.c_void_p(64), ctypes.c_void_p(96), 16, None) == _capi.MBP_EINVAL
    assert b"overlap" in lib.mbp_last_error()


def _bad(lib, mutate_geom=None, mutate_traj=None, cfg=None):
    cfg = cfg or SMALL_CONFIGS["c3_cone256"]
    g = _geometry(cfg)
    traj = {k: (None if v is None else v.copy()) for k, v in config_trajectory(cfg).items()}
    if mutate_geom:
        mutate_geom(g)
    if mutate_traj:
        mutate_traj(traj)
    rc, h = _create(lib, g, traj)
    if rc == 0:
        lib.mbp_plan_destroy(h)
    return rc, lib.mbp_last_error().decode()


def test_validation_error_codes(lib):
    E = _capi
    # enums and shapes
    assert _bad(lib, lambda g: setattr(g, "beam", 5))[0] == E.MBP_EINVAL
    assert _bad(lib, lambda g: setattr(g, "layout", 3))[0] == E.MBP_EINVAL
    assert _bad(lib, lambda g: setattr(g, "D", 0))[0] == E.MBP_EINVAL
    assert _bad(lib, lambda g: setattr(g, "views", 0))[0] == E.MBP_EINVAL
    assert _bad(lib, lambda g: setattr(g, "du", -1.0))[0] == E.MBP_EINVAL
    c1 = CONFIGS["c1_parallel2d"]
    assert _bad(lib, lambda g: setattr(g, "rows", 2), cfg=c1)[0] == E.MBP_EINVAL
    assert _bad(lib, lambda g: setattr(g, "layout", 1), cfg=c1)[0] == E.MBP_EINVAL
    # non-finite geometry
    rc, msg = _bad(lib, mutate_traj=lambda t: t["src"].__setitem__((3, 1), np.nan))
    assert rc == E.MBP_ENONFINITE and "finite" in msg
    assert _bad(lib, mutate_traj=lambda t: t["ev"].__setitem__((0, 2), np.inf))[0] == E.MBP_ENONFINITE
    assert _bad(lib, lambda g: g.spacing.__setitem__(1, float("nan")))[0] == E.MBP_ENONFINITE
    assert _bad(lib, lambda g: g.center.__setitem__(0, float("inf")))[0] == E.MBP_ENONFINITE
    # pitch range and ratio
    rc, msg = _bad(lib, lambda g: g.spacing.__setitem__(0, 1e-7))
    assert rc == E.MBP_ERANGE and "1e-6" in msg
    assert _bad(lib, lambda g: g.spacing.__setitem__(2, 2e6))[0] == E.MBP_ERANGE
    rc, msg = _bad(lib, lambda g: (g.spacing.__setitem__(0, 1e-3), g.spacing.__setitem__(1, 20.0)))
    assert rc == E.MBP_ERANGE and "1e4" in msg
    # source on a pixel, zero axes, parallel axes
    def on_pixel(t):
        t["src"][2] = t["det"][2]
    rc, msg = _bad(lib, mutate_traj=on_pixel)
    assert rc == E.MBP_ECOINCIDENT and "must differ" in msg
    assert _bad(lib, mutate_traj=lambda t: t["eu"].__setitem__(1, 0.0))[0] == E.MBP_ECOINCIDENT
    assert _bad(lib, mutate_traj=lambda t: t["ev"].__setitem__(1, t["eu"][1]))[0] == E.MBP_ECOINCIDENT
    assert _bad(lib, mutate_traj=lambda t: t["src"].__setitem__(0, 0.0), cfg=c1)[0] == E.MBP_ECOINCIDENT
    # near and far geometry
    def near(t):
        t["src"][4] = t["det"][4] + 1e-9 * np.cross(t["eu"][4], t["ev"][4])
    rc, msg = _bad(lib, mutate_traj=near)
    assert rc == E.MBP_ERANGE and "1e6" in msg
    rc, msg = _bad(lib, mutate_traj=lambda t: t["src"].__setitem__((5, 0), 2e15))
    assert rc == E.MBP_ERANGE and "1e15" in msg
    # a source in the detector plane but off the pixel array is fine
    def in_plane_off_array(t):
        t["src"][6] = t["det"][6] + 1e4 * t["eu"][6]
    assert _bad(lib, mutate_traj=in_plane_off_array)[0] == 0
    # 2^31-element arrays
    assert _bad(lib, lambda g: (setattr(g, "D", 2048), setattr(g, "H", 1024), setattr(g, "W", 1024)))[0] == E.MBP_ETOOLARGE
    assert _bad(lib, lambda g: (setattr(g, "rows", 1 << 16), setattr(g, "cols", 1 << 16)))[0] == E.MBP_ETOOLARGE
    # missing trajectory arrays
    g = _geometry(SMALL_CONFIGS["c3_cone256"])
    h = ctypes.c_void_p()
    assert lib.mbp_plan_create(ctypes.byref(g), None, None, None, None, ctypes.byref(h)) == E.MBP_EINVAL
    assert lib.mbp_plan_create(None, None, None, None, None, ctypes.byref(h)) == E.MBP_EINVAL


def test_parallel3d_plans_and_errors(lib):
    """The 3-D parallel beam: a circular trajectory with rows along z takes the column walk in
    either layout, a tilted one the generic walk; a missing row axis, a zero ray direction and
    a non-finite direction are refused."""
    from tests.test_hostcheck import parallel3d_config
    from workloads import random_parallel_3d_trajectory
    E = _capi
    cfg = parallel3d_config()
    for layout in ("DHW", "WHD"):
        rc, h = _create(lib, _geometry(cfg, layout), config_trajectory(cfg))
        assert rc == 0
        inf = _info(lib, h)
        assert inf.column_capable == 1 and inf.path == 2
        lib.mbp_plan_destroy(h)
    rc, h = _create(lib, _geometry(cfg), random_parallel_3d_trajectory(cfg.views, seed=2))
    assert rc == 0 and _info(lib, h).column_capable == 0
    lib.mbp_plan_destroy(h)
    # rays along z: the column walk has no xy line to share
    t = config_trajectory(cfg)
    t["src"][3] = (0.0, 0.0, 1.0)
    t["eu"][3] = (1.0, 0.0, 0.0)
    t["ev"][3] = (0.0, 1.0, 0.0)
    rc, h = _create(lib, _geometry(cfg), t)
    assert rc == 0 and _info(lib, h).column_capable == 0
    lib.mbp_plan_destroy(h)
    assert _bad(lib, mutate_traj=lambda t: t.__setitem__("ev", None), cfg=cfg)[0] == E.MBP_EINVAL
    rc, msg = _bad(lib, mutate_traj=lambda t: t["src"].__setitem__(2, 0.0), cfg=cfg)
    assert rc == E.MBP_ECOINCIDENT and "must differ" in msg
    assert _bad(lib, mutate_traj=lambda t: t["src"].__setitem__((1, 2), np.nan), cfg=cfg)[0] == E.MBP_ENONFINITE
    # no source: no near-geometry refusal for a detector anywhere along the rays
    assert _bad(lib, mutate_traj=lambda t: t["det"].__setitem__(0, (1e3, 0.0, 0.0)), cfg=cfg)[0] == 0


def test_solver_workspace_and_argument_checks(lib):
    """mbp_cgls_workspace_size follows its stated layout; mbp_normal and mbp_cgls refuse bad
    arguments with their status before any device work; batch 0 does nothing."""
    E = _capi
    cfg = SMALL_CONFIGS["c3_cone256"]
    rc, h = _create(lib, _geometry(cfg), config_trajectory(cfg))
    assert rc == 0
    n = ctypes.c_size_t()
    P = ctypes.c_void_p

    def up(b):
        return (b + 255) // 256 * 256
    for batch, iters in ((1, 0), (2, 10), (3, 7)):
        assert lib.mbp_cgls_workspace_size(h, batch, iters, ctypes.byref(n)) == 0
        want = (2 * up(batch * cfg.n_rays * 4) + 2 * up(batch * cfg.n_voxels * 4)
                + up(batch * 8 * 8) + up(batch * (iters + 1) * 8) + up(batch * 512 * 8))
        assert n.value == want
    assert lib.mbp_cgls_workspace_size(h, 0, 5, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.mbp_cgls_workspace_size(h, -1, 5, ctypes.byref(n)) == E.MBP_EINVAL
    assert lib.mbp_cgls_workspace_size(h, 1, -1, ctypes.byref(n)) == E.MBP_EINVAL
    assert lib.mbp_cgls_workspace_size(None, 1, 1, ctypes.byref(n)) == E.MBP_EINVAL
    fake = P(1 << 20)            # never dereferenced: every call below fails validation
    hist = (ctypes.c_double * 4)()
    assert lib.mbp_cgls(None, fake, 1, fake, 3, 0.0, fake, 1 << 40, hist, None) == E.MBP_EINVAL
    assert lib.mbp_cgls(h, fake, -1, fake, 3, 0.0, fake, 1 << 40, hist, None) == E.MBP_EINVAL
    assert lib.mbp_cgls(h, fake, 1, fake, -2, 0.0, fake, 1 << 40, hist, None) == E.MBP_EINVAL
    assert lib.mbp_cgls(h, fake, 1, fake, 3, -1.0, fake, 1 << 40, hist, None) == E.MBP_EINVAL
    assert lib.mbp_cgls(h, fake, 1, fake, 3, float("nan"), fake, 1 << 40, hist, None) == E.MBP_EINVAL
    assert lib.mbp_cgls(h, None, 1, fake, 3, 0.0, fake, 1 << 40, hist, None) == E.MBP_EINVAL
    assert lib.mbp_cgls(h, fake, 1, fake, 3, 0.0, P(1 << 20 | 8), 1 << 40, hist, None) == E.MBP_EINVAL
    rc = lib.mbp_cgls(h, fake, 1, fake, 3, 0.0, fake, 1024, hist, None)
    assert rc == E.MBP_ENOMEM and "workspace" in lib.mbp_last_error().decode()
    assert lib.mbp_cgls(h, None, 0, None, 3, 0.0, None, 0, None, None) == 0
    assert lib.mbp_normal(h, None, 1, fake, fake, None) == E.MBP_EINVAL
    assert lib.mbp_normal(h, fake, 1, fake, fake, None) == E.MBP_EINVAL     # out aliases volume
    assert lib.mbp_normal(h, fake, -1, fake, P(1 << 21), None) == E.MBP_EINVAL
    assert lib.mbp_normal(h, None, 0, None, None, None) == 0
    lib.mbp_plan_destroy(h)


def test_python_plan_maps_errors_and_shapes():
    import matched_backprojection_amd as mbp
    cfg = SMALL_CONFIGS["c4_cone512_aniso"]
    traj = config_trajectory(cfg)
    plan = mbp.Plan("cone", cfg.shape, cfg.spacing, traj, (cfg.rows, cfg.cols), (cfg.dv, cfg.du),
                    layout="WHD")
    assert plan.sino_shape == (cfg.views, cfg.rows, cfg.cols)
    assert plan.info["path"] == "column"
    sino = gather_sino_floats(cfg)
    assert plan.workspace_size(1) == 4 * sino
    assert plan.workspace_size(3) == 2 * (cfg.n_voxels + sino) * 4
    plan.set_adjoint("scatter")
    assert plan.workspace_size(1) == 0 and plan.workspace_size(3) == 2 * cfg.n_voxels * 4
    plan.set_adjoint("auto")
    bad = dict(traj)
    bad["src"] = traj["src"].copy()
    bad["src"][0, 0] = np.nan
    with pytest.raises(ValueError, match="finite"):
        mbp.Plan("cone", cfg.shape, cfg.spacing, bad, (cfg.rows, cfg.cols), (cfg.dv, cfg.du))
    with pytest.raises(ValueError):
        mbp.Plan("cone", cfg.shape, (1.0, 1e-9, 1.0), traj, (cfg.rows, cfg.cols))
    p2 = mbp.Plan("parallel", (64, 64), 1.0, config_trajectory(CONFIGS["c1_parallel2d"]), 96, 1.0)
    assert p2.sino_shape == (90, 96) and p2.info["path"] == "generic"
    plan.close()
    p2.close()


def _full_circle_parallel3d(views):
    """A 3-D parallel beam over a full turn (view k along angle 2 pi k / views)."""
    t = np.arange(views, dtype=np.float64) * (2.0 * np.pi / views)
    c, s, zero = np.cos(t), np.sin(t), np.zeros(views)
    return {"src": np.stack([c, s, zero], axis=1), "det": np.zeros((views, 3)),
            "eu": np.stack([-s, c, zero], axis=1), "ev": np.tile([0.0, 0.0, 1.0], (views, 1))}


def _views(traj, order):
    return {k: (None if v is None else np.ascontiguousarray(np.asarray(v)[order])) for k, v in traj.items()}


def test_turn_symmetry_of_the_views(lib):
    """Plan creation finds the turn symmetry that the gather shares cell crossings over: a
    quarter turn for a full circle of 4k views on a square grid of equal x and y pitch centred
    on the turn's axis (anticlockwise or clockwise), a half turn for 2k views or a grid that is
    not square, none for an odd view count, an off-centre grid, an odd W, a short scan, views
    out of angular order or a 3-D parallel beam over half a turn (view v + V/2 is then a
    quarter turn of view v, which pairs no cells). Host logic only."""
    from dataclasses import replace
    base = SMALL_CONFIGS["c4_cone512_aniso"]

    def orbit(cfg, traj=None, center=None):
        g = _geometry(cfg)
        if center is not None:
            g.center[0], g.center[1], g.center[2] = center
        rc, h = _create(lib, g, config_trajectory(cfg) if traj is None else traj)
        assert rc == 0, lib.mbp_last_error()
        inf = _info(lib, h)
        assert inf.last_adjoint_orbit == 0 and inf.last_forward_orbit == 0
        lib.mbp_plan_destroy(h)
        return inf.orbit

    c48 = replace(base, views=48)
    assert orbit(c48) == 4
    assert orbit(c48, traj=_views(config_trajectory(c48), np.arange(48)[::-1])) == 4   # clockwise
    assert orbit(replace(base, views=46)) == 2
    assert orbit(replace(base, views=45)) == 1
    assert orbit(replace(c48, shape=(48, 64, 48))) == 2          # W != H
    assert orbit(replace(c48, spacing=(1.5, 1.0, 1.25))) == 2    # dx != dy
    assert orbit(replace(c48, shape=(48, 63, 63))) == 1          # odd W
    assert orbit(c48, center=(3.0, 0.0, 0.0)) == 1               # axis off the grid's centre
    assert orbit(c48, center=(0.0, 0.0, 7.0)) == 4               # z offsets keep the symmetry
    perm = np.random.default_rng(3).permutation(48)
    assert orbit(c48, traj=_views(config_trajectory(c48), perm)) == 1
    short = replace(base, views=80)
    assert orbit(replace(base, views=40), traj=_views(config_trajectory(short), np.arange(40))) == 1
    p3 = replace(c48, beam="parallel3d", trajectory="parallel3d")
    assert orbit(p3) == 1
    assert orbit(p3, traj=_full_circle_parallel3d(48)) == 4
    # the switch: 0 or 1 only
    rc, h = _create(lib, _geometry(c48), config_trajectory(c48))
    assert rc == 0
    assert lib.mbp_plan_set_orbit(h, 0) == 0 and lib.mbp_plan_set_orbit(h, 1) == 0
    assert lib.mbp_plan_set_orbit(h, 2) == _capi.MBP_EINVAL
    assert lib.mbp_plan_set_orbit(None, 1) == _capi.MBP_EINVAL
    lib.mbp_plan_destroy(h)
