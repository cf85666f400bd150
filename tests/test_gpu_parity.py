"""GPU parity: the HIP path against the fp64 oracle, through the C ABI (runs on the GPU machine).

Bar (per configuration and batch member): relative L2 error <= 1e-5; max relative error
<= 1e-4 per ray / voxel, where the relative error of element i is
|g_i - o_i| / max(|o_i|, 1e-6 * max|o|); adjoint identity |<Ax, y> - <x, A^T y>| / |<Ax, y>|
<= 1e-5 with fp64 dot products of the GPU's fp32 outputs. Rays that miss the volume box must
be exactly 0.

Reduced twins of the five configurations are compared element by element in full; the
full-size configurations are compared on sampled rays and voxels that the oracle computes
one by one (forward: Siddon on the chosen rays; adjoint: the chord definition at the chosen
voxels), plus the adjoint identity over the whole arrays.
"""

import numpy as np
import pytest

from workloads import (CONFIGS, SMALL_CONFIGS, add_noise, config_phantom, config_trajectory,
                       random_cone_trajectory, sinogram_field)
from workloads.configs import CONTEXT_CONFIGS

pytestmark = pytest.mark.gpu

RTOL_L2 = 1e-5
RTOL_MAX = 1e-4
RTOL_ADJ = 1e-5


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch, torch.device("cuda:0")


@pytest.fixture(scope="module")
def mbp():
    import matched_backprojection_amd as m
    return m


def say(msg):
    print(msg, flush=True)


def rel_l2(g, o):
    return float(np.linalg.norm((g - o).ravel()) / np.linalg.norm(o.ravel()))


def max_rel(g, o):
    floor = 1e-6 * float(np.abs(o).max())
    return float((np.abs(g - o) / np.maximum(np.abs(o), floor)).max())


def check(g, o, what):
    e2, em = rel_l2(g, o), max_rel(g, o)
    say(f"  {what}: rel-L2 {e2:.2e}  max-rel {em:.2e}")
    assert e2 <= RTOL_L2, (what, e2)
    assert em <= RTOL_MAX, (what, em)


def geom_of(cfg):
    return {"beam": cfg.beam, "shape": cfg.shape, "spacing": cfg.spacing, "views": cfg.views,
            "rows": cfg.rows, "cols": cfg.cols, "du": cfg.du, "dv": cfg.dv}


def make_plan(mbp, cfg, traj=None, layout=None):
    traj = config_trajectory(cfg) if traj is None else traj
    if cfg.beam in ("cone", "parallel3d"):
        return mbp.Plan(cfg.beam, cfg.shape, cfg.spacing, traj, (cfg.rows, cfg.cols),
                        (cfg.dv, cfg.du), layout=layout or cfg.layout)
    return mbp.Plan(cfg.beam, cfg.shape, cfg.spacing, traj, cfg.cols, cfg.du)


def to_device_volume(torch, dev, x, layout):
    """numpy (B?, D, H, W) -> device tensor of the same shape in the given layout."""
    if layout == "DHW" or x.ndim == 2:
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    perm = (2, 1, 0) if x.ndim == 3 else (0, 3, 2, 1)
    t = torch.from_numpy(np.ascontiguousarray(x.transpose(perm))).to(dev)
    return t.permute(perm)


def paths_of(cfg):
    return ["column", "generic"] if cfg.beam == "cone" else ["generic"]


# ------------------------------------------------------------------------------------------
# Reduced configurations: full element-by-element comparison


@pytest.mark.parametrize("name", list(SMALL_CONFIGS))
def test_small_config_parity(torch_dev, mbp, oracle, name):
    torch, dev = torch_dev
    cfg = SMALL_CONFIGS[name]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    x = config_phantom(cfg)
    ref, counts = oracle.project(geom, traj, x, counts=True)
    missed = counts == 0                  # rays that do not enter the volume box
    y = ref.astype(np.float32)
    if cfg.noise_sigma:
        y = add_noise(y, cfg.noise_sigma, cfg.noise_seed)
    bref = oracle.backproject(geom, traj, y)
    for path in paths_of(cfg):
        say(f"case {cfg.name} path={path} layout={cfg.layout} batch={cfg.batch}")
        plan = make_plan(mbp, cfg)
        plan.set_path(path)
        xd = to_device_volume(torch, dev, x, cfg.layout)
        p = plan.project(xd).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        members = range(cfg.batch) if cfg.batch else [None]
        for m in members:
            g, o = (p, ref) if m is None else (p[m], ref[m])
            check(g, o, f"forward member {m}")
            assert np.all(g[missed] == 0.0), "rays that miss the volume must be exactly 0"
        yd = torch.from_numpy(y).to(dev)
        b = plan.backproject(yd)
        torch.cuda.synchronize()
        bn = b.cpu().numpy().astype(np.float64)
        for m in members:
            g, o = (bn, bref) if m is None else (bn[m], bref[m])
            check(g, o, f"adjoint member {m}")
        # adjoint identity on the GPU pair
        lhs = float(np.dot(p.ravel(), y.astype(np.float64).ravel()))
        rhs = float(np.dot(x.astype(np.float64).ravel(), bn.ravel()))
        say(f"  adjoint identity {abs(lhs - rhs) / abs(lhs):.2e}")
        assert abs(lhs - rhs) <= RTOL_ADJ * abs(lhs)
        plan.close()


@pytest.mark.parametrize("trajectory", ["circular", "circular_tilted"])
def test_steep_cone_parity(torch_dev, mbp, oracle, trajectory):
    """Rows crossing several z cells per xy cell and leaving through the box's z faces: the
    gather's general piece walk, in both its plain-LDS and its atomic mode; with the detector
    tilted, the per-row gather's piece walk and its LDS atomics for units whose cells are out
    of order."""
    from dataclasses import replace
    from tests.test_hostcheck import steep_cone_config
    torch, dev = torch_dev
    cfg = replace(steep_cone_config(), trajectory=trajectory)
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(21)
    x = rng.random(cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    y = rng.random(ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    for adjoint in ("gather", "scatter"):
        say(f"case steep cone, adjoint={adjoint}")
        plan = make_plan(mbp, cfg)
        plan.set_adjoint(adjoint)
        p = plan.project(to_device_volume(torch, dev, x, cfg.layout)).cpu().numpy().astype(np.float64)
        check(p, ref, "forward")
        b = plan.backproject(torch.from_numpy(y).to(dev)).cpu().numpy().astype(np.float64)
        check(b, bref, "adjoint")
        plan.close()


@pytest.mark.parametrize("flip", [False, True])
def test_tall_detector_parity(torch_dev, mbp, oracle, flip):
    """Eight rows per lane: the gather's fast fixed-point form (pairs of z cells per row,
    rows far above and below the volume discarded), for one volume and batches of two and
    four interleaved members, with detector rows running up or down."""
    from tests.test_hostcheck import flipped, tall_detector_config
    torch, dev = torch_dev
    cfg = tall_detector_config()
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    if flip:
        traj = flipped(traj)
    rng = np.random.default_rng(31)
    x = rng.random(cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    ys = rng.random((4,) + ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    plan = make_plan(mbp, cfg, traj=traj)
    assert plan.info["path"] == "column"
    say(f"case tall detector flip={flip} forward")
    p = plan.project(to_device_volume(torch, dev, x, cfg.layout)).cpu().numpy().astype(np.float64)
    check(p, ref, "forward")
    for B in (0, 2, 4):
        say(f"case tall detector flip={flip} adjoint B={B}")
        yd = torch.from_numpy(ys[0] if B == 0 else ys[:B]).to(dev)
        b = plan.backproject(yd).cpu().numpy().astype(np.float64)
        if B == 0:
            check(b, bref[0], "adjoint")
        for m in range(B):
            check(b[m], bref[m], f"adjoint member {m}")
    plan.close()


@pytest.mark.parametrize("flip", [False, True])
def test_short_detector_parity(torch_dev, mbp, oracle, flip):
    """Eight rows per lane with every ray inside the volume's z range (512 rows at 0.1 pitch):
    every fast item keeps to the column (the host replay's fast_inside check accepts all of
    them), so the gather writes their cell pairs without clamping, for one volume and
    batches of two and four interleaved members, with detector rows running up or down."""
    from tests.test_hostcheck import flipped, short_detector_config
    torch, dev = torch_dev
    cfg = short_detector_config()
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    if flip:
        traj = flipped(traj)
    rng = np.random.default_rng(37)
    x = rng.random(cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    ys = rng.random((4,) + ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    plan = make_plan(mbp, cfg, traj=traj)
    assert plan.info["path"] == "column"
    say(f"case short detector flip={flip} forward")
    p = plan.project(to_device_volume(torch, dev, x, cfg.layout)).cpu().numpy().astype(np.float64)
    check(p, ref, "forward")
    for B in (0, 2, 4):
        say(f"case short detector flip={flip} adjoint B={B}")
        yd = torch.from_numpy(ys[0] if B == 0 else ys[:B]).to(dev)
        b = plan.backproject(yd).cpu().numpy().astype(np.float64)
        if B == 0:
            check(b, bref[0], "adjoint")
        for m in range(B):
            check(b[m], bref[m], f"adjoint member {m}")
    plan.close()


@pytest.mark.parametrize("flip", [False, True])
def test_helical_runs_parity(torch_dev, mbp, oracle, flip):
    """The helical twin (one row per lane): its lanes share cell pairs in runs that the gather
    combines across the wave before writing, along the wave when the detector rows run up and
    against it when they run down; for one volume and batches of two and four members."""
    from tests.test_hostcheck import flipped
    torch, dev = torch_dev
    cfg = SMALL_CONFIGS["c5_helical_b4"]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    if flip:
        traj = flipped(traj)
    rng = np.random.default_rng(37)
    x = rng.random(cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    ys = rng.random((4,) + ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    plan = make_plan(mbp, cfg, traj=traj)
    assert plan.info["path"] == "column"
    say(f"case helical runs flip={flip} forward")
    p = plan.project(to_device_volume(torch, dev, x, cfg.layout)).cpu().numpy().astype(np.float64)
    check(p, ref, "forward")
    for B in (0, 2, 4):
        say(f"case helical runs flip={flip} adjoint B={B}")
        yd = torch.from_numpy(ys[0] if B == 0 else ys[:B]).to(dev)
        b = plan.backproject(yd).cpu().numpy().astype(np.float64)
        if B == 0:
            check(b, bref[0], "adjoint")
        for m in range(B):
            check(b[m], bref[m], f"adjoint member {m}")
    plan.close()


@pytest.mark.parametrize("rows", [150, 200, 300])
def test_mid_detector_parity(torch_dev, mbp, oracle, rows):
    """Three, four and five rows per lane (the gather loads four rows per lane for three and
    four, six for five; rows past a lane's own are loaded and ignored), unbatched and with a
    batch of four."""
    from dataclasses import replace
    from tests.test_hostcheck import tall_detector_config
    torch, dev = torch_dev
    cfg = replace(tall_detector_config(), rows=rows, name=f"c4m_rows{rows}")
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(rows)
    x = rng.random(cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    ys = rng.random((4,) + ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    plan = make_plan(mbp, cfg, traj=traj)
    assert plan.info["path"] == "column"
    say(f"case mid detector rows={rows} forward")
    p = plan.project(to_device_volume(torch, dev, x, cfg.layout)).cpu().numpy().astype(np.float64)
    check(p, ref, "forward")
    for B in (0, 4):
        say(f"case mid detector rows={rows} adjoint B={B}")
        yd = torch.from_numpy(ys[0] if B == 0 else ys[:B]).to(dev)
        b = plan.backproject(yd).cpu().numpy().astype(np.float64)
        if B == 0:
            check(b, bref[0], "adjoint")
        for m in range(B):
            check(b[m], bref[m], f"adjoint member {m}")
    plan.close()


def test_parallel3d_parity(torch_dev, mbp, oracle):
    """3-D parallel beam (infinite lines): circular with detector rows along z (column walk
    with the gather adjoint, and the generic walk), random directions with tilted detectors
    (generic walk), in both layouts, unbatched and with a batch of three."""
    from tests.test_hostcheck import parallel3d_config
    from workloads import random_parallel_3d_trajectory
    torch, dev = torch_dev
    cfg = parallel3d_config()
    geom = geom_of(cfg)
    rng = np.random.default_rng(41)
    xs = rng.random((3,) + cfg.shape).astype(np.float32)
    cases = ((config_trajectory(cfg), ("column", "generic"), "circular"),
             (random_parallel_3d_trajectory(cfg.views, seed=6, offset=3.0), ("generic",), "random"))
    for traj, paths, label in cases:
        ref = oracle.project(geom, traj, xs)
        ys = rng.random(ref.shape).astype(np.float32)
        bref = oracle.backproject(geom, traj, ys)
        for layout in ("DHW", "WHD"):
            plan = make_plan(mbp, cfg, traj=traj, layout=layout)
            for path in paths:
                plan.set_path(path)
                for B in (0, 3):
                    say(f"case parallel3d {label} layout={layout} path={path} B={B}")
                    x_in = xs[0] if B == 0 else xs
                    p = plan.project(to_device_volume(torch, dev, x_in, layout)).cpu().numpy().astype(np.float64)
                    y_in = ys[0] if B == 0 else ys
                    b = plan.backproject(torch.from_numpy(y_in).to(dev)).cpu().numpy().astype(np.float64)
                    for m in range(max(B, 1)):
                        g_p, g_b = (p, b) if B == 0 else (p[m], b[m])
                        check(g_p, ref[m], f"forward member {m}")
                        check(g_b, bref[m], f"adjoint member {m}")
            plan.close()


def test_lattice_aligned_parity(torch_dev, mbp, oracle):
    """Lines that meet two or three grid planes at once (exact ties between x, y and z
    crossings; see lattice_parallel3d): column walk (counted z crossings, the general per-cell
    form for the (1, 1, 1) lines) and generic walk, forward and adjoint, both layouts."""
    from tests.test_hostcheck import lattice_parallel3d
    torch, dev = torch_dev
    geom, traj = lattice_parallel3d()
    rng = np.random.default_rng(23)
    x = rng.random(geom["shape"]).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    y = rng.random(ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    for layout in ("DHW", "WHD"):
        plan = mbp.Plan("parallel3d", geom["shape"], geom["spacing"], traj, (geom["rows"], geom["cols"]),
                        (geom["dv"], geom["du"]), layout=layout)
        for path in ("column", "generic"):
            plan.set_path(path)
            say(f"case lattice-aligned lines layout={layout} path={path}")
            p = plan.project(to_device_volume(torch, dev, x, layout)).cpu().numpy().astype(np.float64)
            b = plan.backproject(torch.from_numpy(y).to(dev)).cpu().numpy().astype(np.float64)
            check(p, ref, "forward")
            check(b, bref, "adjoint")
        plan.close()


def test_general_trajectory_parity(torch_dev, mbp, oracle):
    """Random tilted frames (row axis not parallel to z), anisotropic grid: the generic walk
    forward; adjoint by the per-ray gather (rows that do not keep their cells in order along
    the wave fall back to LDS atomics) and by the generic walk's global atomics."""
    torch, dev = torch_dev
    cfg = SMALL_CONFIGS["c4_cone512_aniso"]
    traj = random_cone_trajectory(30, seed=12, radius=150.0, sdd=260.0, tilt=0.5)
    from dataclasses import replace
    cfg = replace(cfg, views=30)
    geom = geom_of(cfg)
    x = config_phantom(cfg)
    ref = oracle.project(geom, traj, x)
    y = np.random.default_rng(3).random(ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    say("case random tilted cone trajectory (generic walk)")
    plan = make_plan(mbp, cfg, traj=traj)
    assert plan.info["path"] == "generic"
    p = plan.project(to_device_volume(torch, dev, x, cfg.layout)).cpu().numpy().astype(np.float64)
    check(p, ref, "forward")
    for kind in ("gather", "scatter"):
        say(f"case random tilted cone trajectory adjoint={kind}")
        plan.set_adjoint(kind)
        b = plan.backproject(torch.from_numpy(y).to(dev)).cpu().numpy().astype(np.float64)
        check(b, bref, f"adjoint {kind}")
    plan.close()


@pytest.mark.parametrize("layout", ["DHW", "WHD"])
def test_tilted_circular_parity(torch_dev, mbp, oracle, layout):
    """A circular cone whose detector is rotated by a few degrees in its plane (rows not
    along z): the generic walk forward, with threads taking consecutive columns (DHW volume)
    or consecutive rows (z-fastest volume); adjoint by the per-ray gather and by the generic
    walk's atomics; unbatched and with batches of two and four, rows running up or down."""
    from dataclasses import replace
    from tests.test_hostcheck import flipped
    torch, dev = torch_dev
    cfg = replace(SMALL_CONFIGS["c3_cone256"], trajectory="circular_tilted", layout=layout)
    geom = geom_of(cfg)
    rng = np.random.default_rng(41)
    xs = rng.random((4,) + cfg.shape).astype(np.float32)
    for flip in (False, True):
        traj = config_trajectory(cfg)
        if flip:
            traj = flipped(traj)
        ref = oracle.project(geom, traj, xs)
        ys = rng.random(ref.shape).astype(np.float32)
        bref = oracle.backproject(geom, traj, ys)
        plan = make_plan(mbp, cfg, traj=traj)
        assert plan.info["path"] == "generic"
        for B in (0, 2, 4):
            x_in = xs[0] if B == 0 else xs[:B]
            say(f"case tilted circular cone layout={layout} flip={flip} B={B} forward")
            p = plan.project(to_device_volume(torch, dev, x_in, layout)).cpu().numpy().astype(np.float64)
            for m in range(max(B, 1)):
                check(p if B == 0 else p[m], ref[m], f"forward member {m}")
            y_in = ys[0] if B == 0 else ys[:B]
            for kind in ("gather", "scatter"):
                if flip and kind == "scatter":
                    continue
                say(f"case tilted circular cone layout={layout} flip={flip} B={B} adjoint={kind}")
                plan.set_adjoint(kind)
                b = plan.backproject(torch.from_numpy(y_in).to(dev)).cpu().numpy().astype(np.float64)
                for m in range(max(B, 1)):
                    check(b if B == 0 else b[m], bref[m], f"adjoint {kind} member {m}")
            plan.set_adjoint("gather")
        plan.close()


@pytest.mark.parametrize("case", ["quarter", "quarter_clockwise", "half", "half_rect",
                                  "parallel3d_quarter"])
def test_orbit_pair_parity(torch_dev, mbp, oracle, case):
    """The pair shared over a turn symmetry of the views (one walk gives the P rays of the
    views V / P apart; one gather crossing serves the P cells of an orbit): the plan finds the
    symmetry, both operators take it in both layouts (the gather also when adding into a
    volume, the forward also per member of a batch), and they match the oracle, the unshared
    operators (to fp32 rounding) and the adjoint identity."""
    from tests.test_hostcheck import _turn_cases
    torch, dev = torch_dev
    cfg, traj, P, turn = _turn_cases()[case]
    geom = geom_of(cfg)
    x = config_phantom(cfg)
    ref = oracle.project(geom, traj, x)
    y = np.random.default_rng(5).random((cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    pre = np.random.default_rng(6).random(cfg.shape).astype(np.float32)
    for layout in ("WHD", "DHW"):
        say(f"case orbit {case} (P={P}, turn {turn}) layout={layout}")
        plan = make_plan(mbp, cfg, traj=traj, layout=layout)
        assert plan.info["orbit"] == P
        yd = torch.from_numpy(y).to(dev)
        b = plan.backproject(yd).cpu().numpy().astype(np.float64)
        assert plan.info["last_adjoint_orbit"] == P and plan.info["last_adjoint"] == "gather"
        check(b, bref, "orbit gather")
        out = to_device_volume(torch, dev, pre, layout)
        plan.backproject(yd, out=out, accumulate=True)
        check(out.cpu().numpy().astype(np.float64), bref + pre.astype(np.float64), "orbit accumulate")
        xd = to_device_volume(torch, dev, x, layout)
        p = plan.project(xd).cpu().numpy().astype(np.float64)
        assert plan.info["last_forward_orbit"] == P
        check(p, ref, "orbit forward")
        lhs = float(np.dot(p.ravel(), y.astype(np.float64).ravel()))
        rhs = float(np.dot(x.astype(np.float64).ravel(), b.ravel()))
        say(f"  adjoint identity {abs(lhs - rhs) / abs(lhs):.2e}")
        assert abs(lhs - rhs) <= RTOL_ADJ * abs(lhs)
        # a batch of three: an interleaved pair, then the last member alone, which alone takes
        # the symmetry
        x3 = np.stack([x, 0.5 * x, x[::-1].copy()]).astype(np.float32)
        p3 = plan.project(to_device_volume(torch, dev, x3, layout)).cpu().numpy().astype(np.float64)
        assert plan.info["last_forward_orbit"] == 1
        check(p3[2], oracle.project(geom, traj, x3[2]), "orbit forward, batch member 2")
        plan.set_orbit(False)
        b1 = plan.backproject(yd).cpu().numpy().astype(np.float64)
        p1 = plan.project(xd).cpu().numpy().astype(np.float64)
        assert plan.info["last_adjoint_orbit"] == 1 and plan.info["last_forward_orbit"] == 1
        check(b1, bref, "unshared gather")
        check(p1, ref, "unshared forward")
        d, df = rel_l2(b, b1), rel_l2(p, p1)
        say(f"  shared vs unshared rel-L2: adjoint {d:.2e}, forward {df:.2e}")
        assert d <= 1e-6 and df <= 1e-6
        plan.close()


@pytest.mark.parametrize("case", ["tilted_quarter", "tilted_quarter_clockwise", "tilted_half",
                                  "fan_quarter", "fan_half"])
def test_orbit_generic_walk_and_per_row_gather_parity(torch_dev, mbp, oracle, case):
    """Geometries off the column walk with a turn symmetry: the generic forward walk shares
    each walk over it (turned element strides), and the per-row gather (the cone tilted in its
    detector plane) each cell clip; the 2-D fan's adjoint is the generic walk's atomics, which
    do not share. Both layouts for the cone, the accumulating gather, against the oracle, the
    unshared operators and the adjoint identity."""
    from tests.test_hostcheck import _generic_turn_cases
    torch, dev = torch_dev
    cfg, traj, P, turn = _generic_turn_cases()[case]
    geom = geom_of(cfg)
    x = np.random.default_rng(8).random(cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    y = np.random.default_rng(9).random(ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    cone = cfg.beam == "cone"
    for layout in (("WHD", "DHW") if cone else ("DHW",)):
        say(f"case generic orbit {case} (P={P}, turn {turn}) layout={layout}")
        plan = make_plan(mbp, cfg, traj=traj, layout=layout)
        assert plan.info["orbit"] == P and plan.info["path"] == "generic"
        xd = to_device_volume(torch, dev, x, layout)
        yd = torch.from_numpy(y).to(dev)
        p = plan.project(xd).cpu().numpy().astype(np.float64)
        assert plan.info["last_forward_orbit"] == P
        check(p, ref, "shared generic forward")
        b = plan.backproject(yd).cpu().numpy().astype(np.float64)
        assert plan.info["last_adjoint_orbit"] == (P if cone else 1)
        check(b, bref, "per-row gather" if cone else "generic adjoint")
        if cone:
            pre = np.random.default_rng(10).random(cfg.shape).astype(np.float32)
            out = to_device_volume(torch, dev, pre, layout)
            plan.backproject(yd, out=out, accumulate=True)
            check(out.cpu().numpy().astype(np.float64), bref + pre.astype(np.float64), "accumulate")
        lhs = float(np.dot(p.ravel(), y.astype(np.float64).ravel()))
        rhs = float(np.dot(x.astype(np.float64).ravel(), b.ravel()))
        say(f"  adjoint identity {abs(lhs - rhs) / abs(lhs):.2e}")
        assert abs(lhs - rhs) <= RTOL_ADJ * abs(lhs)
        plan.set_orbit(False)
        p1 = plan.project(xd).cpu().numpy().astype(np.float64)
        b1 = plan.backproject(yd).cpu().numpy().astype(np.float64)
        assert plan.info["last_forward_orbit"] == 1 and plan.info["last_adjoint_orbit"] == 1
        d, df = rel_l2(b, b1), rel_l2(p, p1)
        say(f"  shared vs unshared rel-L2: adjoint {d:.2e}, forward {df:.2e}")
        assert df <= 1e-6 and d <= 1e-6
        plan.close()


def test_view_batches_layouts_batches_and_accumulate(torch_dev, mbp, oracle):
    """Ragged view batches, both layouts, batch sizes 0..5, accumulation, caller workspace."""
    torch, dev = torch_dev
    cfg = SMALL_CONFIGS["c3_cone256"]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(8)
    xs = rng.random((5,) + cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, xs)
    ys = rng.random(ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    for layout in ("DHW", "WHD"):
        for path in ("column", "generic"):
            plan = make_plan(mbp, cfg, layout=layout)
            plan.set_path(path)
            plan.set_view_batch(7)            # 36 views -> launches of 7 + ragged 1
            for B in (0, 1, 3, 5):
                say(f"case view-batch 7 layout={layout} path={path} B={B}")
                xd = to_device_volume(torch, dev, xs[:B], layout)
                p = plan.project(xd).cpu().numpy().astype(np.float64)
                assert p.shape == (B, cfg.views, cfg.rows, cfg.cols)
                for m in range(B):
                    check(p[m], ref[m], f"forward member {m}")
                b = plan.backproject(torch.from_numpy(ys[:B]).to(dev)).cpu().numpy().astype(np.float64)
                assert b.shape == (B,) + cfg.shape
                for m in range(B):
                    check(b[m], bref[m], f"adjoint member {m}")
            # accumulate into a prefilled volume, unbatched
            pre = rng.random(cfg.shape).astype(np.float32)
            out = to_device_volume(torch, dev, pre, layout)
            plan.backproject(torch.from_numpy(ys[0]).to(dev), out=out, accumulate=True)
            check(out.cpu().numpy().astype(np.float64), bref[0] + pre.astype(np.float64), "accumulate")
            plan.close()
    # a caller-owned workspace gives the same result; a too-small one is refused
    plan = make_plan(mbp, cfg)
    need = plan.workspace_size(5)
    from tests.test_capi import gather_sino_floats
    assert need == 4 * (cfg.n_voxels + gather_sino_floats(cfg)) * 4
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev)
    plan.set_workspace(ws)
    p = plan.project(torch.from_numpy(xs).to(dev)).cpu().numpy().astype(np.float64)
    for m in range(5):
        check(p[m], ref[m], f"caller workspace member {m}")
    plan.set_workspace(torch.empty(16, dtype=torch.float32, device=dev))
    with pytest.raises(mbp.MbpError):
        plan.project(torch.from_numpy(xs).to(dev))
    plan.close()


def test_tilted_view_batches_and_accumulate(torch_dev, mbp, oracle):
    """The per-row gather over ragged view batches (each launch adds into the previous ones),
    both layouts, batches of one, three and five members (groups of four and one), and
    accumulation into a prefilled volume."""
    from dataclasses import replace
    torch, dev = torch_dev
    cfg = replace(SMALL_CONFIGS["c3_cone256"], trajectory="circular_tilted")
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(9)
    ys = rng.random((5, cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    for layout in ("DHW", "WHD"):
        plan = make_plan(mbp, cfg, traj=traj, layout=layout)
        plan.set_view_batch(7)                # 36 views -> launches of 7 + ragged 1
        for B in (1, 3, 5):
            say(f"case tilted view-batch 7 layout={layout} B={B}")
            b = plan.backproject(torch.from_numpy(ys[:B]).to(dev)).cpu().numpy().astype(np.float64)
            for m in range(B):
                check(b[m], bref[m], f"adjoint member {m}")
        pre = rng.random(cfg.shape).astype(np.float32)
        out = to_device_volume(torch, dev, pre, layout)
        plan.backproject(torch.from_numpy(ys[0]).to(dev), out=out, accumulate=True)
        check(out.cpu().numpy().astype(np.float64), bref[0] + pre.astype(np.float64), "accumulate")
        plan.close()


@pytest.mark.parametrize("trajectory", ["circular", "circular_tilted"])
def test_z_chunked_gathers_parity(torch_dev, mbp, oracle, trajectory):
    """A column too tall for one wave's LDS (600 cells of four interleaved members, more than
    the 2048 floats a wave holds): the gathers split it into z chunks of 512 cells, each wave
    building its items for its own chunk (rows 460, eight per lane, fast cell pairs on the
    circle; per-row clips when tilted); one member fits a single chunk."""
    from dataclasses import replace
    torch, dev = torch_dev
    cfg = replace(SMALL_CONFIGS["c4_cone512_aniso"], name="tall_column", shape=(600, 8, 8),
                  spacing=(0.5, 1.0, 1.0), sid=400.0, sdd=600.0, rows=460, cols=24, views=8,
                  trajectory=trajectory, layout="DHW")
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(17)
    ys = rng.random((4, cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    plan = make_plan(mbp, cfg, traj=traj)
    for B in (1, 4):
        say(f"case z-chunked {trajectory} B={B}")
        b = plan.backproject(torch.from_numpy(ys[:B]).to(dev)).cpu().numpy().astype(np.float64)
        for m in range(B):
            check(b[m], bref[m], f"adjoint member {m}")
    plan.close()


def test_layout_conversion_roundtrip(torch_dev, mbp):
    torch, dev = torch_dev
    x = torch.rand((3, 37, 41, 29), device=dev)
    w = mbp.convert_layout(x, to_whd=True)
    assert w.stride()[1:] == (1, 37, 37 * 41)
    assert torch.equal(w, x)                       # same logical tensor
    back = mbp.convert_layout(w, to_whd=False)
    assert back.is_contiguous() and torch.equal(back, x)


def test_segment_counts_match_oracle(torch_dev, mbp, oracle):
    torch, dev = torch_dev
    for name in ("c2_fan2d", "c3_cone256", "c5_helical_b4"):
        cfg = SMALL_CONFIGS[name]
        geom, traj = geom_of(cfg), config_trajectory(cfg)
        x = np.zeros(cfg.shape, np.float32)
        _, cnt = oracle.project(geom, traj, x, counts=True)
        for path in paths_of(cfg):
            say(f"case segment count {cfg.name} path={path}")
            plan = make_plan(mbp, cfg)
            plan.set_path(path)
            n = plan.segment_count()
            say(f"  gpu {n} oracle {int(cnt.sum())}")
            assert abs(n - int(cnt.sum())) <= 1e-3 * cnt.sum()
            plan.close()


# ------------------------------------------------------------------------------------------
# Full-size configurations: sampled rays and voxels, adjoint identity


def _unit_columns(cfg, rng):
    """(view, column) pairs whose whole detector column (every row) is compared: the forward
    kernel's unit of work is 64 rows of one column of one view, so whole columns cover every
    unit of them, ragged last unit included; first, middle and last columns of the first view,
    a view a quarter turn on, and two random views with random columns."""
    views = [0, cfg.views // 4 + 3] + [int(v) for v in rng.integers(0, cfg.views, 2)]
    cols = [0, cfg.cols // 2, cfg.cols - 1]
    pairs = [(v, j) for v in views[:2] for j in cols]
    pairs += [(v, int(j)) for v in views[2:] for j in rng.integers(0, cfg.cols, 3)]
    return pairs


def _sample_rays(cfg, n, rng):
    per_view = cfg.rows * cfg.cols
    ids = [rng.integers(0, cfg.n_rays, n)]
    v = int(rng.integers(cfg.views))
    ids.append(v * per_view + (cfg.rows - 1) * cfg.cols + np.arange(0, cfg.cols, 7))   # last row
    for view, col in _unit_columns(cfg, rng):                                          # columns
        ids.append(view * per_view + np.arange(cfg.rows) * cfg.cols + col)
    return np.unique(np.concatenate(ids))


def _unit_z_columns(cfg):
    """(x, y) of the xy cells whose whole z column is compared: the gathers' unit of work is
    one z column, and their cells are dealt in tiles (32 x 32 for both gathers when the grid
    holds them, else 16 x 32; with a turn symmetry, tiles of the quadrant or half whose cells
    stand for the orbits; earlier tilings took 64 x 8 and 8 x 8, whose edges stay sampled);
    the columns sit on the volume's faces, on both sides of the first tile edges of every
    tiling in x and y, on both sides of the midlines where the orbits' images meet, and on the
    images of those cells."""
    D, H, W = cfg.shape
    xs = sorted({min(x, W - 1) for x in (0, 15, 16, 31, 32, 63, 64, W - 1)})
    ys = sorted({min(y, H - 1) for y in (0, 7, 8, 31, 32, H - 1)})
    cells = {(x, y) for x in xs for y in ys}
    for x, y in ((7, 7), (8, 8), (7, 8), (W // 2 - 1, H // 2 - 1), (W // 2, H // 2),
                 (W // 2 - 1, H // 2), (W // 2, H // 2 - 1)):
        for cx, cy in ((x, y), (W - 1 - x, H - 1 - y), (W - 1 - y, x), (y, W - 1 - x)):
            if 0 <= cx < W and 0 <= cy < H:
                cells.add((cx, cy))
    return sorted(cells)


def _sample_voxels(cfg, n, rng):
    ids = [rng.integers(0, cfg.n_voxels, n)]
    shape = cfg.shape
    corners = np.array(np.meshgrid(*[[0, s - 1] for s in shape], indexing="ij")).reshape(len(shape), -1)
    ids.append(np.ravel_multi_index(corners, shape))
    if len(shape) == 3:
        D, H, W = shape
        for x, y in _unit_z_columns(cfg):
            ids.append((np.arange(D) * H + y) * W + x)
    return np.unique(np.concatenate(ids))


def _full_size_config(name):
    """A full-size configuration by name: the five configurations, the pages' context
    workload, and the 256^3 cone with its detector rotated in its plane (rows not along z;
    volume z-fastest), the timed workload of the per-row gather."""
    from dataclasses import replace
    if name == "c3_cone256_tilted":
        return replace(CONFIGS["c3_cone256"], name=name, trajectory="circular_tilted", layout="WHD")
    return CONFIGS.get(name) or CONTEXT_CONFIGS[name]


@pytest.mark.parametrize("name", list(CONFIGS) + list(CONTEXT_CONFIGS) + ["c3_cone256_tilted"])
def test_full_size_parity(torch_dev, mbp, oracle, name):
    torch, dev = torch_dev
    cfg = _full_size_config(name)
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(100 + len(name))
    x = config_phantom(cfg)
    small = cfg.n_rays * 1000 < 5e8         # c1, c2: the oracle runs the whole operator
    plan = make_plan(mbp, cfg)
    say(f"case full-size {cfg.name} path={plan.info['path']} layout={cfg.layout} batch={cfg.batch}")
    xd = to_device_volume(torch, dev, x, cfg.layout)
    p_dev = plan.project(xd)
    torch.cuda.synchronize()
    members = list(range(cfg.batch)) if cfg.batch else [None]
    if small:
        ref = oracle.project(geom, traj, x)
        check(p_dev.cpu().numpy().astype(np.float64), ref, "forward (all rays)")
        y = ref.astype(np.float32)
        if cfg.noise_sigma:
            y = add_noise(y, cfg.noise_sigma, cfg.noise_seed)
    else:
        ids = _sample_rays(cfg, 3000, rng)
        ref = oracle.project_rays(geom, traj, x, ids)
        flat = p_dev.reshape((cfg.batch or 1), -1)[:, torch.from_numpy(ids).to(dev)].cpu().numpy()
        for m in members:
            g = flat[0 if m is None else m].astype(np.float64)
            o = ref if m is None else ref[m]
            check(g, o, f"forward member {m} ({ids.size} sampled rays)")
        y = sinogram_field(tuple(p_dev.shape), seed=7)
    yd = torch.from_numpy(y).to(dev)
    b_dev = plan.backproject(yd)
    torch.cuda.synchronize()
    if small:
        bref = oracle.backproject(geom, traj, y)
        check(b_dev.cpu().numpy().astype(np.float64), bref, "adjoint (all voxels)")
    else:
        vids = _sample_voxels(cfg, 400, rng)
        bref = oracle.backproject_voxels(geom, traj, y, vids)
        bflat = b_dev.reshape((cfg.batch or 1), -1) if cfg.layout == "DHW" else \
            b_dev.contiguous().reshape((cfg.batch or 1), -1)
        g_all = bflat[:, torch.from_numpy(vids).to(dev)].cpu().numpy().astype(np.float64)
        for m in members:
            check(g_all[0 if m is None else m], bref if m is None else bref[m],
                  f"adjoint member {m} ({vids.size} sampled voxels)")
    # adjoint identity over the whole arrays (fp64 dot products of fp32 outputs)
    pv = p_dev.double()
    lhs = torch.dot(pv.reshape(-1), yd.double().reshape(-1)).item()
    rhs = torch.dot(xd.double().contiguous().reshape(-1), b_dev.double().contiguous().reshape(-1)).item()
    say(f"  adjoint identity {abs(lhs - rhs) / abs(lhs):.2e}")
    assert abs(lhs - rhs) <= RTOL_ADJ * abs(lhs)
    plan.close()
    del p_dev, b_dev, xd, yd
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------------------
# Volumes of 2 GiB or more: the forward's buffer resource per cell


def _whd_on_device(torch, dev, x):
    """numpy (B?, D, H, W) in C order -> a device tensor of the same shape with z-fastest
    strides (the transpose runs on the device: a host transpose of 2 GiB takes many seconds)."""
    t = torch.from_numpy(x).to(dev)
    perm = (2, 1, 0) if x.ndim == 3 else (0, 3, 2, 1)
    return t.permute(perm).contiguous().permute(perm)


def _check_rays(plan_out, cfg, geom, traj, x, ids, oracle, torch, dev, label):
    ref = oracle.project_rays(geom, traj, x, ids)
    B = x.shape[0] if x.ndim == 4 else 1
    flat = plan_out.reshape(B, -1)[:, torch.from_numpy(ids).to(dev)].cpu().numpy().astype(np.float64)
    for m in range(B):
        check(flat[m], ref if x.ndim == 3 else ref[m], f"{label} member {m} ({ids.size} rays)")


def test_interleaved_batch_over_2gib_forward_parity(torch_dev, mbp, oracle):
    """The 512^3 cone with a batch of four: the interleaved pass holds 2 GiB, more than one
    buffer resource's 31-bit offsets span, so the forward bases a resource at every cell's
    column (the four-member variant). Sampled rays and whole detector columns of several
    views against the oracle, for every member."""
    torch, dev = torch_dev
    cfg = CONFIGS["c4_cone512_aniso"]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(71)
    x = np.empty((4,) + cfg.shape, np.float32)
    x[0] = config_phantom(cfg)
    for m in range(1, 4):
        x[m] = rng.random(cfg.shape, dtype=np.float32)
    plan = make_plan(mbp, cfg)
    assert plan.info["path"] == "column" and plan.info["members_per_pass"] == 4
    assert 4 * cfg.n_voxels * 4 >= 2 ** 31
    say("case c4 batch 4 (interleaved pass of 2 GiB) forward")
    xd = _whd_on_device(torch, dev, x)
    p = plan.project(xd)
    torch.cuda.synchronize()
    ids = _sample_rays(cfg, 2000, rng)
    _check_rays(p, cfg, geom, traj, x, ids, oracle, torch, dev, "forward")
    plan.close()
    del xd, p
    torch.cuda.empty_cache()


def test_single_volume_over_2gib_parity(torch_dev, mbp, oracle):
    """One 512 x 1024 x 1024 volume (2 GiB, z-fastest): the one-member forward with a buffer
    resource per cell, and the gather writing a column of a volume beyond 2^31 bytes; the
    detector (96 rows: a ragged second wave) covers the whole grid. Sampled rays and whole
    detector columns, sampled voxels and whole z columns against the oracle, and the adjoint
    identity over the whole arrays."""
    from dataclasses import replace
    torch, dev = torch_dev
    cfg = replace(CONFIGS["c4_cone512_aniso"], name="cone_2gib", shape=(512, 1024, 1024),
                  spacing=(1.0, 1.0, 1.0), sid=2000.0, sdd=3000.0, views=16, rows=96, cols=192,
                  du=8.0, dv=8.0, layout="WHD", background=0.0)
    assert cfg.n_voxels * 4 >= 2 ** 31
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(73)
    say("case single 2 GiB volume: drawing the volume")
    xw = rng.random(cfg.shape[::-1], dtype=np.float32)        # (W, H, D): z fastest
    xd = torch.from_numpy(xw).to(dev).permute(2, 1, 0)          # (D, H, W) view, z-fastest strides
    del xw
    x = xd.contiguous().cpu().numpy()                           # C-order (D, H, W) for the oracle
    plan = make_plan(mbp, cfg)
    assert plan.info["path"] == "column"
    say("case single 2 GiB volume forward")
    p = plan.project(xd)
    torch.cuda.synchronize()
    ids = _sample_rays(cfg, 2000, rng)
    _check_rays(p, cfg, geom, traj, x, ids, oracle, torch, dev, "forward")
    say("case single 2 GiB volume adjoint")
    y = rng.random((cfg.views, cfg.rows, cfg.cols), dtype=np.float32)
    yd = torch.from_numpy(y).to(dev)
    b = plan.backproject(yd)
    torch.cuda.synchronize()
    vids = _sample_voxels(cfg, 400, rng)
    bref = oracle.backproject_voxels(geom, traj, y, vids)
    g = b.permute(2, 1, 0).reshape(-1)          # the (W, H, D) storage, flat
    D, H, W = cfg.shape
    z, rem = np.divmod(vids, H * W)
    yy, xx = np.divmod(rem, W)
    store = (xx * H + yy) * D + z
    gv = g[torch.from_numpy(store).to(dev)].cpu().numpy().astype(np.float64)
    check(gv, bref, f"adjoint ({vids.size} sampled voxels)")
    lhs = torch.dot(p.double().reshape(-1), yd.double().reshape(-1)).item()
    rhs = torch.dot(xd.permute(2, 1, 0).double().reshape(-1), b.permute(2, 1, 0).double().reshape(-1)).item()
    say(f"  adjoint identity {abs(lhs - rhs) / abs(lhs):.2e}")
    assert abs(lhs - rhs) <= RTOL_ADJ * abs(lhs)
    plan.close()
    del xd, p, b, yd
    torch.cuda.empty_cache()


def test_segment_count_full_size_oblique_views(torch_dev, mbp, oracle):
    """The metric's numerator at full size: the counting kernel over 24 oblique views of the
    512^3 cone (every 30th view from view 7, at 3.5 + 15 k degrees) against the oracle's
    exact count of positive-length segments on the same views.

    Bound: the kernel counts segments longer than eps = 1e-6 of the smallest pitch, with
    lengths formed from fp64 crossing distances (accurate to far below eps), so it can only
    miss the oracle's pieces in (0, eps]: a plane crossing of one axis that falls within eps
    of another axis' crossing. Crossings of axis a lie p_a / |c_a| apart along the ray
    (c_a the direction component per unit of the walk's parameter; |c_x|, |c_y| <= 1, and
    |c_z| < 0.2 with p_z = 1.5 here), so each crossing meets such a neighbour with probability
    at most 2 eps (1/p_x + 1/p_y + |c_z|/p_z) < 4.3e-6; the count may fall short of the
    oracle's by at most 1e-5 of it (over 2x that rate), and never exceed it."""
    torch, dev = torch_dev
    cfg = CONFIGS["c4_cone512_aniso"]
    full = config_trajectory(cfg)
    sel = 7 + 30 * np.arange(24)
    traj = {k: (None if v is None else np.ascontiguousarray(v[sel])) for k, v in full.items()}
    from dataclasses import replace
    sub = replace(cfg, views=24)
    geom = geom_of(sub)
    say("case segment count, c4 at full size, 24 oblique views")
    plan = make_plan(mbp, sub, traj=traj)
    n = plan.segment_count()
    _, cnt = oracle.project(geom, traj, np.zeros(sub.shape, np.float32), counts=True)
    o = int(cnt.sum())
    say(f"  gpu {n} oracle {o} short by {(o - n) / o:.2e}")
    assert n <= o
    assert o - n <= 1e-5 * o
    plan.close()


# ------------------------------------------------------------------------------------------
# The gather in view batches sized to its workspace


@pytest.mark.parametrize("trajectory", ["circular", "circular_tilted"])
def test_gather_in_view_batches_of_a_small_workspace(torch_dev, mbp, oracle, trajectory):
    """A caller workspace that holds the volume part and five views' share of the reordered
    sinogram: the gather (column or per-row) runs in launches of five views (36 views: seven
    of five and a ragged one), each adding into the previous ones; unbatched (z-fastest volume
    used in place, so the workspace is all sinogram) and with a batch of four (interleaved
    volume in the workspace too). A workspace below one view's share is refused."""
    from dataclasses import replace
    torch, dev = torch_dev
    cfg = replace(SMALL_CONFIGS["c3_cone256"], trajectory=trajectory, layout="WHD")
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(53)
    ys = rng.random((4, cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bref = oracle.backproject(geom, traj, ys)
    for B in (1, 4):
        plan = make_plan(mbp, cfg, traj=traj)
        plan.set_view_batch(5)
        need = plan.workspace_size(B)
        plan.set_view_batch(1)
        least = plan.workspace_size(B)
        plan.set_view_batch(0)
        assert plan.workspace_size(B) > need > least > 0
        ws = torch.empty(need // 4, dtype=torch.float32, device=dev)
        plan.set_workspace(ws)
        say(f"case gather in view batches {trajectory} B={B}")
        y_in = ys[0] if B == 1 else ys
        b = plan.backproject(torch.from_numpy(y_in).to(dev)).cpu().numpy().astype(np.float64)
        info = plan.info
        say(f"  {info['last_adjoint']} on the {info['last_adjoint_walk']} walk, "
            f"{info['last_adjoint_views_per_launch']} views per launch")
        assert info["last_adjoint"] == "gather" and info["last_adjoint_views_per_launch"] == 5
        for m in range(B):
            check(b if B == 1 else b[m], bref[m], f"adjoint member {m}")
        # the forward with the same workspace: the walk and the members it served are reported
        vol = plan.empty_volume(None if B == 1 else B, device=dev)
        vol.fill_(1.0)
        plan.project(vol)
        torch.cuda.synchronize()
        info = plan.info
        say(f"  forward on the {info['last_forward_walk']} walk, "
            f"{info['last_forward_members_per_pass']} members per pass")
        if trajectory == "circular":
            assert info["last_forward_walk"] == "column" and info["last_forward_members_per_pass"] == B
        else:
            assert info["last_forward_walk"] == "generic" and info["last_forward_members_per_pass"] == 0
        plan.set_workspace(torch.empty((least - 4) // 4, dtype=torch.float32, device=dev))
        with pytest.raises(mbp.MbpError):
            plan.backproject(torch.from_numpy(y_in).to(dev))
        plan.close()


def test_gather_under_the_memory_rule_at_full_size(torch_dev, mbp, oracle):
    """The 512^3 cone's adjoint with nearly all device memory held elsewhere: one call may
    use at most a quarter of the free memory, so the library's workspace holds only a few
    dozen views of the reordered sinogram and the gather runs in many launches (before, this
    case fell back to the atomic scatter, 38 times slower). Whole z columns and sampled voxels
    against the oracle."""
    torch, dev = torch_dev
    cfg = CONFIGS["c4_cone512_aniso"]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(59)
    y = sinogram_field((cfg.views, cfg.rows, cfg.cols), seed=11)
    yd = torch.from_numpy(y).to(dev)
    plan = make_plan(mbp, cfg)
    out = plan.empty_volume(device=dev)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    hold = torch.empty(max(free - (256 << 20), 0), dtype=torch.uint8, device=dev)
    say(f"case gather under the memory rule: {hold.numel() / 2**30:.1f} GiB held, "
        f"{torch.cuda.mem_get_info()[0] / 2**20:.0f} MiB free")
    plan.backproject(yd, out=out)
    torch.cuda.synchronize()
    del hold
    torch.cuda.empty_cache()
    info = plan.info
    say(f"  {info['last_adjoint']} on the {info['last_adjoint_walk']} walk, "
        f"{info['last_adjoint_views_per_launch']} views per launch")
    assert info["last_adjoint"] == "gather" and info["last_adjoint_walk"] == "column"
    assert 1 <= info["last_adjoint_views_per_launch"] < cfg.views
    vids = _sample_voxels(cfg, 200, rng)
    bref = oracle.backproject_voxels(geom, traj, y, vids)
    g = out.contiguous().reshape(-1)[torch.from_numpy(vids).to(dev)].cpu().numpy().astype(np.float64)
    check(g, bref, f"adjoint ({vids.size} sampled voxels)")
    plan.close()
    del yd, out
    torch.cuda.empty_cache()
