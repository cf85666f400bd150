"""GPU parity of the normal operator and CGLS against the fp64 oracle (marked gpu).

The normal operator is held to the pair's bar (rel-L2 <= 1e-5, max-rel <= 1e-4). CGLS
iterates are held to RTOL_CGLS_X in relative L2 and the residual histories to RTOL_CGLS_R of
||r0||: the GPU runs the same recurrences with fp32 vectors and fp64 norms and step sizes,
so its iterates differ from the fp64 ones by the operators' fp32 rounding (about 1e-7
relative per product) carried through the few iterations run here. Measured on MI355X:
iterates within 4e-7, histories within 3e-9 of ||r0||; the bounds leave 25x and 30x room.
"""

import numpy as np
import pytest

from tests.test_gpu_parity import check, geom_of, make_plan, say, to_device_volume
from workloads import SMALL_CONFIGS, config_phantom, config_trajectory, random_cone_trajectory

pytestmark = pytest.mark.gpu

RTOL_CGLS_X = 1e-5
RTOL_CGLS_R = 1e-7


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch, torch.device("cuda:0")


@pytest.fixture(scope="module")
def mbp():
    import matched_backprojection_amd as m
    return m


def _to_numpy(t):
    return t.detach().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["c4_cone512_aniso", "c3_cone256"])
def test_normal_operator_parity(torch_dev, mbp, oracle, name):
    """A^T A x on the GPU (column walk with the gather, caller's layout) against the fp64
    oracle, unbatched and with a batch of two."""
    torch, dev = torch_dev
    cfg = SMALL_CONFIGS[name]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    rng = np.random.default_rng(17)
    xs = rng.random((2,) + cfg.shape).astype(np.float32)
    ref = oracle.normal(geom, traj, xs.astype(np.float64))
    plan = make_plan(mbp, cfg)
    for B in (0, 2):
        say(f"case normal operator {cfg.name} layout={cfg.layout} B={B}")
        x_in = xs[0] if B == 0 else xs
        sino = torch.empty(((B,) if B else ()) + plan.sino_shape, dtype=torch.float32, device=dev)
        out = plan.normal(to_device_volume(torch, dev, x_in, cfg.layout), sinogram=sino)
        got = _to_numpy(out)
        for m in range(max(B, 1)):
            check(got if B == 0 else got[m], ref[m], f"normal member {m}")
        # the sinogram it filled on the way is A x
        sref = oracle.project(geom, traj, x_in)
        check(_to_numpy(sino), sref, "A x")
    plan.close()


def _noisy_data(oracle, geom, traj, cfg, seed):
    x_true = config_phantom(cfg)
    if x_true.ndim == 4:
        x_true = x_true[0]
    y = oracle.project(geom, traj, x_true)
    rng = np.random.default_rng(seed)
    return (y + 0.01 * np.abs(y).max() * rng.standard_normal(y.shape)).astype(np.float32)


def _check_cgls(x_gpu, h_gpu, x_ref, h_ref, what):
    ex = np.linalg.norm(x_gpu - x_ref) / np.linalg.norm(x_ref)
    eh = np.abs(h_gpu - h_ref).max() / h_ref[0]
    say(f"  {what}: iterate rel-L2 {ex:.2e}, residual history {eh:.2e} of ||r0||")
    assert ex <= RTOL_CGLS_X, (what, ex)
    assert eh <= RTOL_CGLS_R, (what, eh)


def test_cgls_parity_from_zero(torch_dev, mbp, oracle):
    """Eight CGLS iterations on the anisotropic small cone, volumes kept z-fastest."""
    torch, dev = torch_dev
    cfg = SMALL_CONFIGS["c4_cone512_aniso"]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    y = _noisy_data(oracle, geom, traj, cfg, seed=3)
    x_ref, h_ref = oracle.cgls(geom, traj, y, 8)
    assert np.all(np.diff(h_ref) < 0)
    plan = make_plan(mbp, cfg)
    say("case CGLS from zero, 8 iterations")
    x, h = plan.cgls(torch.from_numpy(y).to(dev), 8)
    _check_cgls(_to_numpy(x), h, x_ref, h_ref, "CGLS")
    plan.close()


def test_cgls_batch_start_and_threshold(torch_dev, mbp, oracle):
    """Two members solved together: member 0 from zero with a residual threshold that stops
    it after a few iterations, member 1 from a nonzero start; each equals its own oracle
    solve. The threshold lies halfway (geometrically) between two of the oracle's residual
    norms, so fp32 rounding cannot move the stopping iteration."""
    torch, dev = torch_dev
    cfg = SMALL_CONFIGS["c3_cone256"]
    geom, traj = geom_of(cfg), config_trajectory(cfg)
    y0 = _noisy_data(oracle, geom, traj, cfg, seed=4)
    y1 = (0.5 * y0 + np.random.default_rng(5).random(y0.shape)).astype(np.float32)
    x1_start = np.random.default_rng(6).random(cfg.shape).astype(np.float32)
    iters = 6
    _, h_full = oracle.cgls(geom, traj, y0, iters)
    rtol = float(np.sqrt(h_full[3] * h_full[4]) / np.linalg.norm(y0.astype(np.float64)))
    x_ref0, h_ref0 = oracle.cgls(geom, traj, y0, iters, rtol=rtol)
    assert np.all(h_ref0[4:] == h_ref0[4]) and h_ref0[3] > h_ref0[4]
    x_ref1, h_ref1 = oracle.cgls(geom, traj, y1, iters, x0=x1_start.astype(np.float64), rtol=rtol)
    assert h_ref1[-1] > rtol * np.linalg.norm(y1.astype(np.float64))   # member 1 never stops
    plan = make_plan(mbp, cfg)
    say(f"case CGLS batch of 2, x0 and rtol {rtol:.3e}, layout={cfg.layout}")
    x0 = to_device_volume(torch, dev, np.stack([np.zeros(cfg.shape, np.float32), x1_start]), cfg.layout)
    x, h = plan.cgls(torch.from_numpy(np.stack([y0, y1])).to(dev), iters, x0=x0, rtol=rtol)
    assert x.data_ptr() == x0.data_ptr()
    xn = _to_numpy(x)
    _check_cgls(xn[0], h[0], x_ref0, h_ref0, "member 0 (stops)")
    assert np.all(h[0][4:] == h[0][4])
    _check_cgls(xn[1], h[1], x_ref1, h_ref1, "member 1 (from x0)")
    plan.close()


def test_cgls_generic_walk(torch_dev, mbp, oracle):
    """CGLS on a tilted-detector trajectory: generic walk with the atomic adjoint."""
    torch, dev = torch_dev
    from dataclasses import replace
    cfg = replace(SMALL_CONFIGS["c4_cone512_aniso"], views=20, layout="DHW")
    traj = random_cone_trajectory(20, seed=12, radius=150.0, sdd=260.0, tilt=0.5)
    geom = geom_of(cfg)
    y = _noisy_data(oracle, geom, traj, cfg, seed=7)
    x_ref, h_ref = oracle.cgls(geom, traj, y, 4)
    plan = make_plan(mbp, cfg, traj=traj)
    assert plan.info["path"] == "generic"
    say("case CGLS generic walk, 4 iterations")
    x, h = plan.cgls(torch.from_numpy(y).to(dev), 4)
    _check_cgls(_to_numpy(x), h, x_ref, h_ref, "CGLS generic")
    plan.close()
