"""CPU replay of the GPU walks: bounds on every launch shape, and the walk logic (no GPU).

The replay compiles the kernels' traversal header for the host. It is not parity (it shares
the GPU path's code); it shows, before anything runs on a GPU, that every cell the walks visit
at the parity and benchmark shapes lies inside the volume, and that the walk logic reproduces
the oracle's line integrals at fp32 rounding level.
"""

import numpy as np
import pytest

from tests import _hostcheck as HC
from workloads import (CONFIGS, SMALL_CONFIGS, config_phantom, config_trajectory,
                       random_cone_trajectory, random_parallel_3d_trajectory)


def _geom(cfg):
    return {"beam": cfg.beam, "shape": cfg.shape, "spacing": cfg.spacing, "views": cfg.views,
            "rows": cfg.rows, "cols": cfg.cols, "du": cfg.du, "dv": cfg.dv}


def _paths(cfg):
    return ["generic", "column"] if cfg.beam in ("cone", "parallel3d") else ["generic"]


def parallel3d_config():
    """A small 3-D parallel beam on a circle (detector rows along z), on the anisotropic grid
    of the small cone twin; rows above and below the volume miss it."""
    from dataclasses import replace
    return replace(SMALL_CONFIGS["c4_cone512_aniso"], name="p3s_parallel3d", beam="parallel3d",
                   layout="DHW", views=30, rows=80, cols=96, du=0.9, dv=1.1)


def lattice_parallel3d():
    """3-D parallel lines through the lattice of a unit grid whose faces lie on integers:
    along (2, 0, 1) and (0, 2, -1) every other x (or y) plane is met exactly where a z plane
    is (pixels at half-integer v); along (1, 1, 0) and (1, 1, 1) x and y planes are met
    together (pixels at half-integer diagonal offsets, du = sqrt 2); (-2, 0, -1) runs the
    first one backwards. Detector rows along z, so the column walk applies."""
    import math
    dirs = [(2.0, 0.0, 1.0), (-2.0, 0.0, -1.0), (0.0, 2.0, -1.0), (1.0, 1.0, 0.0), (1.0, 1.0, 1.0),
            (2.0, 1.0, 0.5)]
    src, det, eu, ev = [], [], [], []
    for d in dirs:
        h = math.hypot(d[0], d[1])
        src.append(d)
        det.append((0.0, 0.0, 0.0))
        eu.append((-d[1] / h, d[0] / h, 0.0))
        ev.append((0.0, 0.0, 1.0))
    traj = {k: np.asarray(v, dtype=np.float64) for k, v in
            (("src", src), ("det", det), ("eu", eu), ("ev", ev))}
    geom = {"beam": "parallel3d", "shape": (16, 12, 20), "spacing": (1.0, 1.0, 1.0),
            "views": len(dirs), "rows": 12, "cols": 16, "du": math.sqrt(2.0), "dv": 1.0}
    return geom, traj


def test_lattice_aligned_lines_reproduce_oracle(oracle):
    """Lines that meet two or three planes at once (exact ties in the walks' crossing
    distances): the forward kernel's chunked column walk with its counted z crossings, and
    both walks' forward and adjoint, replayed on the host, against the oracle."""
    geom, traj = lattice_parallel3d()
    rng = np.random.default_rng(17)
    x = rng.random(geom["shape"]).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    s, viol = HC.project_chunked(geom, traj, x)
    assert viol == 0
    assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6
    assert np.abs(s - ref).max() / np.abs(ref).max() < 1e-5
    y = rng.random(ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    for path in ("generic", "column"):
        p_, _, viol = HC.project(path, geom, traj, x)
        assert viol == 0
        assert np.linalg.norm(p_ - ref) / np.linalg.norm(ref) < 1e-6
        b_, viol = HC.backproject(path, geom, traj, y)
        assert viol == 0
        assert np.linalg.norm(b_ - bref) / np.linalg.norm(bref) < 1e-6


def test_parallel3d_walks_reproduce_oracle(oracle):
    """Infinite parallel rays in 3-D through both walks (circular: column and generic;
    random directions with tilted detectors: generic), forward and adjoint, and the gather."""
    cfg = parallel3d_config()
    geom = _geom(cfg)
    x = config_phantom(cfg)
    for traj, paths in ((config_trajectory(cfg), ["generic", "column"]),
                        (random_parallel_3d_trajectory(cfg.views, seed=6, offset=3.0), ["generic"])):
        ref = oracle.project(geom, traj, x)
        y = np.random.default_rng(1).random(ref.shape).astype(np.float32)
        bref = oracle.backproject(geom, traj, y)
        for path in paths:
            s, _, viol = HC.project(path, geom, traj, x)
            assert viol == 0
            assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6
            b, viol = HC.backproject(path, geom, traj, y)
            assert viol == 0
            assert np.linalg.norm(b - bref) / np.linalg.norm(bref) < 1e-6
        if paths == ["generic", "column"]:
            s, viol = HC.project_chunked(geom, traj, x)
            assert viol == 0
            assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6
            b, viol, _ = HC.gather(geom, traj, y, kernel_shares=False)
            assert viol == 0
            assert np.linalg.norm(b - bref) / np.linalg.norm(bref) < 1e-12
    assert np.abs(ref).max() > 1.0


@pytest.mark.parametrize("name", list(SMALL_CONFIGS))
def test_walks_reproduce_oracle_on_small_configs(oracle, name):
    cfg = SMALL_CONFIGS[name]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    x = config_phantom(cfg)
    if cfg.batch:
        x = x[0]
    ref, cnt = oracle.project(geom, traj, x, counts=True)
    y = np.random.default_rng(1).random(ref.shape).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    for path in _paths(cfg):
        s, k, viol = HC.project(path, geom, traj, x)
        assert viol == 0
        assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6
        assert np.abs(s - ref).max() / np.abs(ref).max() < 1e-5
        # counts differ only where planes cross at one point (a zero-length pair in the oracle
        # may round to a tiny positive length in fp32, or the reverse)
        assert abs(int(k.sum()) - int(cnt.sum())) <= 1e-3 * cnt.sum()
        assert (k == cnt).mean() > 0.95
        b, viol = HC.backproject(path, geom, traj, y)
        assert viol == 0
        assert np.linalg.norm(b - bref) / np.linalg.norm(bref) < 1e-6


def test_generic_walk_on_tilted_detectors_and_inside_sources(oracle):
    """Sources inside the volume, tilted detectors, anisotropic off-centre grid."""
    traj = random_cone_trajectory(12, seed=4, radius=9.0, sdd=40.0, tilt=0.6)
    geom = {"beam": "cone", "shape": (14, 17, 19), "spacing": (1.5, 1.0, 0.75),
            "center": (0.375, -0.25, 0.5), "views": 12, "rows": 23, "cols": 21,
            "du": 1.1, "dv": 0.9}
    x = np.random.default_rng(3).random(geom["shape"]).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    s, _, viol = HC.project("generic", geom, traj, x)
    assert viol == 0
    assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6


def _generic_turn_cases():
    """Scans with a turn symmetry that the generic walk takes (name -> config, trajectory,
    orbit, turn sense): the small cone with its detector tilted in its plane on a square grid
    (quarter turn, both senses) and on the 56 x 48 grid (half turn), and the 2-D fan over a
    full circle with 88 views (quarter turn) and 90 (half turn)."""
    from dataclasses import replace
    from tests.test_capi import _views
    c3 = replace(SMALL_CONFIGS["c3_cone256"], trajectory="circular_tilted")
    sq = replace(c3, shape=(40, 48, 48))
    f88 = replace(SMALL_CONFIGS["c2_fan2d"], views=88)
    f90 = SMALL_CONFIGS["c2_fan2d"]
    return {
        "tilted_quarter": (sq, config_trajectory(sq), 4, 1),
        "tilted_quarter_clockwise": (sq, _views(config_trajectory(sq), np.arange(36)[::-1]), 4, -1),
        "tilted_half": (c3, config_trajectory(c3), 2, 0),
        "fan_quarter": (f88, config_trajectory(f88), 4, 1),
        "fan_half": (f90, config_trajectory(f90), 2, 0),
    }


@pytest.mark.parametrize("case", ["tilted_quarter", "tilted_quarter_clockwise", "tilted_half",
                                  "fan_quarter", "fan_half"])
def test_orbit_generic_walk_reproduces_oracle(oracle, case):
    """The generic walk shared over a turn symmetry (the rays of the first V / P views, each
    walk also summing the turned cells, reached by turned element strides, into the rays of
    the views V / P apart) gives every ray's line integral at fp32 rounding level, all offsets
    in bounds; with the wrong turn sense the shared rays miss by percents."""
    cfg, traj, P, turn = _generic_turn_cases()[case]
    geom = _geom(cfg)
    x = np.random.default_rng(6).random(cfg.shape).astype(np.float32)
    ref = oracle.project(geom, traj, x)
    s, _, viol = HC.project("generic", geom, traj, x, orbit=P, turn=turn)
    assert viol == 0
    assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6
    if P == 4:
        s, _, _ = HC.project("generic", geom, traj, x, orbit=P, turn=-turn)
        assert np.linalg.norm(s - ref) / np.linalg.norm(ref) > 1e-2


def _edge_and_random_rays(cfg, n_random, seed):
    rng = np.random.default_rng(seed)
    per_view = cfg.rows * cfg.cols
    ids = [rng.integers(0, cfg.n_rays, n_random)]
    for v in (0, cfg.views // 4, cfg.views // 2, cfg.views - 1):
        k = np.arange(cfg.rows)
        j = np.arange(cfg.cols)
        for kk in (0, cfg.rows - 1):                       # first and last detector rows
            ids.append(v * per_view + kk * cfg.cols + j)
        for jj in (0, cfg.cols // 2, cfg.cols - 1):        # first, middle and last columns
            ids.append(v * per_view + k * cfg.cols + jj)
    return np.concatenate(ids)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_walks_stay_in_bounds_at_full_size(name):
    cfg = CONFIGS[name]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    ids = _edge_and_random_rays(cfg, 20000, seed=len(name))
    for path in _paths(cfg):
        visits, viol = HC.check_rays(path, geom, traj, ids)
        assert viol == 0, (name, path)
        assert visits > ids.size        # rays really cross the volume


@pytest.mark.parametrize("name", ["c3_cone256", "c4_cone512_aniso", "c5_helical_b4", "steep"])
def test_cell_gather_reproduces_oracle_adjoint(oracle, name):
    """The atomic-free adjoint's enumeration (cells -> views -> crossing columns -> rows ->
    z pieces) is the chord definition. Taken all in the fp64 general form it equals the oracle
    to rounding; with the kernel's own choice of form (fast items in fixed point) it equals it
    to the fixed point's resolution (see test_fast_gather_reproduces_oracle_adjoint). The
    steep cone's rows cross several cells per xy cell, so most of its items are general."""
    cfg = steep_cone_config() if name == "steep" else SMALL_CONFIGS[name]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    y = np.random.default_rng(2).random((cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    floor = 1e-6 * np.abs(bref).max()
    for general_only, tol_l2, tol_max in ((True, 1e-12, 1e-9), (False, 3e-9, 2e-5)):
        b, viol, fast = HC.gather(geom, traj, y, kernel_shares=False, general_only=general_only)
        assert viol == 0
        assert (fast == 0) == general_only
        assert np.linalg.norm(b - bref) / np.linalg.norm(bref) < tol_l2
        assert (np.abs(b - bref) / np.maximum(np.abs(bref), floor)).max() < tol_max


def _turn_cases():
    """Scans with a turn symmetry (name, config, trajectory, orbit, turn sense), on the small
    anisotropic cone: a full circle of 48 views anticlockwise and clockwise (quarter turn), 46
    views (half turn), a non-square grid (half turn), and a 3-D parallel beam over a full turn."""
    from dataclasses import replace
    from tests.test_capi import _full_circle_parallel3d, _views
    base = SMALL_CONFIGS["c4_cone512_aniso"]
    c48, c46 = replace(base, views=48), replace(base, views=46)
    rect = replace(c48, shape=(48, 64, 48))
    p3 = replace(c48, beam="parallel3d", trajectory="parallel3d")
    return {
        "quarter": (c48, config_trajectory(c48), 4, 1),
        "quarter_clockwise": (c48, _views(config_trajectory(c48), np.arange(48)[::-1]), 4, -1),
        "half": (c46, config_trajectory(c46), 2, 0),
        "half_rect": (rect, config_trajectory(rect), 2, 0),
        "parallel3d_quarter": (p3, _full_circle_parallel3d(48), 4, 1),
    }


@pytest.mark.parametrize("case", ["quarter", "quarter_clockwise", "half", "half_rect",
                                  "parallel3d_quarter"])
def test_orbit_gather_reproduces_oracle_adjoint(oracle, case):
    """The gather shared over a turn symmetry (items of the first V / P views only, each
    carrying the rows of the views V / P apart into the orbit's other cells) is still the chord
    definition: in the fp64 general form it equals the oracle to rounding, and in the kernel's
    forms to the fixed point's resolution, as the unshared replay does. Replayed with the wrong
    turn sense, the same items land in the wrong cells and miss by percents."""
    cfg, traj, P, turn = _turn_cases()[case]
    geom = _geom(cfg)
    y = np.random.default_rng(2).random((cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    floor = 1e-6 * np.abs(bref).max()
    for general_only, tol_l2, tol_max in ((True, 1e-13, 1e-10), (False, 3e-9, 2e-5)):
        b, viol, fast = HC.gather(geom, traj, y, kernel_shares=False, general_only=general_only,
                                  orbit=P, turn=turn)
        assert viol == 0
        assert (fast == 0) == general_only
        assert np.linalg.norm(b - bref) / np.linalg.norm(bref) < tol_l2
        assert (np.abs(b - bref) / np.maximum(np.abs(bref), floor)).max() < tol_max
    if P == 4:
        b, _, _ = HC.gather(geom, traj, y, general_only=True, orbit=P, turn=-turn)
        assert np.linalg.norm(b - bref) / np.linalg.norm(bref) > 1e-2


def tall_detector_config():
    """The small anisotropic cone with a tall detector (460 rows, so eight rows per lane): the
    gather takes its fast fixed-point form. Most rows pass above or below the volume."""
    from dataclasses import replace
    return replace(SMALL_CONFIGS["c4_cone512_aniso"], name="c4t_tall_detector", rows=460, cols=40,
                   views=12)


def flipped(traj):
    """The same trajectory with detector rows running downwards (z falls as the row grows)."""
    return dict(traj, ev=-traj["ev"])


@pytest.mark.parametrize("flip", [False, True])
def test_fast_gather_reproduces_oracle_adjoint(oracle, flip):
    """The fast form (each lane's rows in fixed point relative to an origin cell, both cells'
    shares from exact integer differences) gives the chord lengths to the fixed point's
    resolution: each end of a row is within 2.5 units of 2^-28 cell (the lane origin rounded to
    nearest, at most four per-row advances each rounded to nearest), which moves a split by at
    most that much; the kernel's fp32 shares add fp32 rounding. Both stay far inside the 1e-4
    per-voxel bar."""
    cfg = tall_detector_config()
    geom, traj = _geom(cfg), config_trajectory(cfg)
    if flip:
        traj = flipped(traj)
    y = np.random.default_rng(5).random((cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    bref = oracle.backproject(geom, traj, y)
    floor = 1e-6 * np.abs(bref).max()
    for kernel_shares, tol_l2, tol_max in ((False, 5e-9, 1e-6), (True, 5e-8, 1e-6)):
        b, viol, fast = HC.gather(geom, traj, y, kernel_shares=kernel_shares)
        assert viol == 0 and fast > 1000
        assert np.linalg.norm(b - bref) / np.linalg.norm(bref) < tol_l2
        assert (np.abs(b - bref) / np.maximum(np.abs(bref), floor)).max() < tol_max


@pytest.mark.parametrize("flip", [False, True])
def test_fast_gather_cell_pairs_never_collide(flip):
    """In the fast form every instruction reads and writes each lane's cell pair {fa, fa + 1}
    without atomics: the pairs of the 64 lanes are disjoint. Adjacent rows in one instruction
    would overlap."""
    cfg = tall_detector_config()
    geom, traj = _geom(cfg), config_trajectory(cfg)
    if flip:
        traj = flipped(traj)
    checked, conflicts, fast = HC.gather_conflicts(geom, traj, mode=0)
    assert fast > 1000 and conflicts == 0
    assert HC.gather_conflicts(geom, traj, mode=2)[1] > 0


@pytest.mark.parametrize("name,flip", [("c3_cone256", False), ("c4_cone512_aniso", False),
                                       ("c5_helical_b4", False), ("c5_helical_b4", True)])
def test_gather_plain_lds_adds_never_collide(name, flip):
    """Where the gather adds into LDS without atomics, the lanes that write together hit
    distinct z cells, and where lanes share a cell pair (runs of lanes, combined across the
    wave before one lane per run writes) every share reaches its cell exactly once. Emulated
    instruction by instruction on these twins, which have one to eight rows per lane, so many
    fast items have such runs; flipped, the runs fall along the wave. Dealing adjacent rows to
    one instruction (with one row per lane, as on the c5 twin, that is the kernel's own
    dealing), writing the runs' cell pairs lane by lane, or shifting the runs one step fewer
    than the kernel fails, so the check has teeth (the c3 twin's runs are single lanes, so
    there the short shift loses nothing)."""
    cfg = SMALL_CONFIGS[name]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    if flip:
        traj = flipped(traj)
    checked, conflicts, fast = HC.gather_conflicts(geom, traj, mode=0)
    assert checked > 10000 and conflicts == 0 and fast == checked
    assert (HC.gather_conflicts(geom, traj, mode=2)[1] > 0) == (name != "c5_helical_b4")
    assert HC.gather_conflicts(geom, traj, mode=3)[1] > 0
    assert (HC.gather_conflicts(geom, traj, mode=4)[1] > 0) == (name != "c3_cone256")


def short_detector_config():
    """The small anisotropic cone with 512 rows at 0.1 pitch (eight rows per lane, no padded
    rows): every row's ray stays inside the volume's z range."""
    from dataclasses import replace
    return replace(SMALL_CONFIGS["c4_cone512_aniso"], name="c4s_short_detector", rows=512, dv=0.1,
                   cols=40, views=12)


@pytest.mark.parametrize("name,zchunk", [("short", None), ("short", 36), ("c3_cone256", None),
                                         ("c5_helical_b4", None), ("c5_helical_b4", 7)])
def test_fast_inside_items_need_no_clamp(name, zchunk):
    """The gather writes a fast item's cell pairs without clamping their indices when
    fast_inside accepts the item for the wave's z chunk. Replayed in the kernel's fixed point
    over every row of every lane (padded rows too), the accepted items' pair indices stay in
    the chunk's range [-2, n + 1], on whole columns and on ragged chunks. With a detector whose
    rays stay inside the volume's z range, every item is accepted on whole columns and many on
    a 36-cell chunk; on the twins whose rays (or padded rows) leave the volume, fewer or none
    are. A test that looks at the first row only lets rows out of chunks."""
    cfg = short_detector_config() if name == "short" else SMALL_CONFIGS[name]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    D = int(cfg.shape[0])
    fast, inside, viol = HC.fast_inside(geom, traj, zchunk or D)
    assert fast > 1000 and viol == 0
    if name == "short":
        assert inside == fast if zchunk is None else inside > fast // 2
    if name == "c5_helical_b4" and zchunk is None:
        assert inside > 0
    if zchunk is not None:
        assert HC.fast_inside(geom, traj, zchunk, mode=1)[2] > 0


def steep_cone_config():
    """A tall, narrow volume next to the source: rows cross several z cells inside one xy cell
    and leave through the bottom and top faces (the gather's general piece walk)."""
    from dataclasses import replace
    return replace(SMALL_CONFIGS["c3_cone256"], name="steep_cone", shape=(100, 20, 20), rows=128,
                   cols=40, dv=3.0, sid=18.0, sdd=40.0, views=6)


def test_gather_steep_rows_walk_aligned():
    """On the steep cone the aligned piece walk stays collision free; the walk that starts at
    the first in-range cell collides."""
    cfg = steep_cone_config()
    geom, traj = _geom(cfg), config_trajectory(cfg)
    checked, conflicts, _ = HC.gather_conflicts(geom, traj, mode=0)
    assert checked > 1000 and conflicts == 0
    assert HC.gather_conflicts(geom, traj, mode=1)[1] > 0
    assert HC.gather_conflicts(geom, traj, mode=2)[1] > 0


@pytest.mark.parametrize("name", ["c3_cone256", "c4_cone512_aniso", "c5_helical_b4"])
def test_gather_plain_lds_adds_never_collide_full_size(name):
    cfg = CONFIGS[name]
    sel = [0, cfg.views // 3, (2 * cfg.views) // 3]
    traj = {k: (None if v is None else v[sel]) for k, v in config_trajectory(cfg).items()}
    geom = dict(_geom(cfg), views=len(sel))
    checked, conflicts, fast = HC.gather_conflicts(geom, traj)
    assert checked > 100000 and conflicts == 0
    assert fast == checked              # every crossing of these geometries takes the fast form


@pytest.mark.parametrize("which", ["c3_cone256", "c4_cone512_aniso", "c5_helical_b4", "steep"])
def test_chunked_column_walk_reproduces_oracle(oracle, which):
    """The forward kernel builds each column's merged xy crossings in chunks of 128 in
    parallel; replayed lane by lane, every chunk position is filled exactly once, all cells
    stay in bounds, and the line integrals match the oracle at fp32 rounding level."""
    cfg = steep_cone_config() if which == "steep" else SMALL_CONFIGS[which]
    geom, traj = _geom(cfg), config_trajectory(cfg)
    x = config_phantom(cfg) if which != "steep" else \
        np.random.default_rng(4).random(cfg.shape).astype(np.float32)
    if x.ndim == 4:
        x = x[0]
    ref = oracle.project(geom, traj, x)
    s, viol = HC.project_chunked(geom, traj, x)
    assert viol == 0
    assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6
    assert np.abs(s - ref).max() / np.abs(ref).max() < 1e-5


@pytest.mark.parametrize("case", ["quarter", "quarter_clockwise", "half", "half_rect",
                                  "parallel3d_quarter"])
def test_orbit_column_walk_reproduces_oracle(oracle, case):
    """The forward shared over a turn symmetry (the walks of the first V / P views, each also
    summing the turned cells into the rays of the views V / P apart): every chunk position and
    turned cell in bounds, every ray's line integral equal to the oracle's at fp32 rounding
    level. With the wrong turn sense the shared rays miss by percents."""
    cfg, traj, P, turn = _turn_cases()[case]
    geom = _geom(cfg)
    x = config_phantom(cfg)
    ref = oracle.project(geom, traj, x)
    s, viol = HC.project_chunked(geom, traj, x, orbit=P, turn=turn)
    assert viol == 0
    assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6
    assert np.abs(s - ref).max() / np.abs(ref).max() < 1e-5
    if P == 4:
        s, _ = HC.project_chunked(geom, traj, x, orbit=P, turn=-turn)
        assert np.linalg.norm(s - ref) / np.linalg.norm(ref) > 1e-2


@pytest.mark.parametrize("name", ["c3_cone256", "c4_cone512_aniso", "c5_helical_b4"])
def test_chunked_column_walk_full_size_views(oracle, name):
    """Full-size columns cross up to ~1000 xy planes, i.e. several chunks: one view each."""
    cfg = CONFIGS[name]
    sel = [cfg.views // 7]
    traj = {k: (None if v is None else v[sel]) for k, v in config_trajectory(cfg).items()}
    geom = dict(_geom(cfg), views=1)
    x = config_phantom(cfg)
    if x.ndim == 4:
        x = x[0]
    ref = oracle.project(geom, traj, x)
    s, viol = HC.project_chunked(geom, traj, x)
    assert viol == 0
    assert np.linalg.norm(s - ref) / np.linalg.norm(ref) < 1e-6


@pytest.mark.parametrize("case", ["tilted", "tilted_flipped", "random", "steep"])
def test_tilt_gather_bands_hold_every_crossing(case):
    """The gather for detectors whose rows do not run along z takes, per view and xy cell, the
    candidate columns and each column's candidate rows from the cell corners' projections. On
    sampled cells every pixel whose ray crosses the cell with positive length (brute force:
    fp64 slab clip of every pixel's ray) lies inside those bands, for a circular cone with its
    detector rotated in its plane (rows up or down) and for random frames; the bands stay
    close to the crossings on the tilted circle."""
    from dataclasses import replace
    from workloads import random_cone_trajectory
    if case == "random":
        cfg = replace(SMALL_CONFIGS["c4_cone512_aniso"], views=30)
        traj = random_cone_trajectory(30, seed=12, radius=150.0, sdd=260.0, tilt=0.5)
    elif case == "steep":
        cfg = replace(steep_cone_config(), trajectory="circular_tilted")
        traj = config_trajectory(cfg)
    else:
        cfg = replace(SMALL_CONFIGS["c3_cone256"], trajectory="circular_tilted")
        traj = config_trajectory(cfg)
        if case == "tilted_flipped":
            traj = flipped(traj)
    hits, misses, cand = HC.tilt_band(_geom(cfg), traj, 3)
    assert hits > 50000 and misses == 0
    if case in ("tilted", "tilted_flipped"):
        assert cand < 1.2 * hits


@pytest.mark.parametrize("case", ["tilted", "tilted_flipped", "random", "steep"])
def test_tilt_gather_replay_reproduces_oracle_adjoint(oracle, case):
    """The gather for detectors whose rows do not run along z, replayed on the CPU unit by
    unit (bands, each row's fp64 clip, two-cell shares or the piece walk, the pre-pass row
    value) gives the oracle's adjoint to fp64 rounding. Every unit whose pair keys are
    monotone along the wave goes through the run combine, replayed on lane sets with the
    kernel's run-length loop and parked lanes, without losing, repeating or misdirecting a
    share; on the tilted circle every unit is monotone (rows up or down), random frames send
    some units to the LDS atomics, and so does the tilted steep cone (rows spanning several
    cells walk their pieces). A combine one shift step short loses shares."""
    from dataclasses import replace
    from workloads import random_cone_trajectory
    if case == "random":
        cfg = replace(SMALL_CONFIGS["c4_cone512_aniso"], views=10)
        traj = random_cone_trajectory(10, seed=12, radius=150.0, sdd=260.0, tilt=0.5)
    elif case == "steep":
        cfg = replace(steep_cone_config(), trajectory="circular_tilted")
        traj = config_trajectory(cfg)
    else:
        cfg = replace(SMALL_CONFIGS["c3_cone256"], trajectory="circular_tilted")
        traj = config_trajectory(cfg)
        if case == "tilted_flipped":
            traj = flipped(traj)
    geom = _geom(cfg)
    y = np.random.default_rng(7).random((cfg.views, cfg.rows, cfg.cols)).astype(np.float32)
    b, units, conflicts, atomic = HC.tilt_gather(geom, traj, y)
    bref = oracle.backproject(geom, traj, y)
    floor = 1e-6 * np.abs(bref).max()
    assert units > 10000 and conflicts == 0
    assert (atomic > 0) == (case in ("random", "steep"))
    assert np.linalg.norm(b - bref) / np.linalg.norm(bref) < 1e-12
    assert (np.abs(b - bref) / np.maximum(np.abs(bref), floor)).max() < 1e-10
    if case in ("tilted", "tilted_flipped"):
        assert HC.tilt_gather(geom, traj, y, mode=1)[2] > 0
