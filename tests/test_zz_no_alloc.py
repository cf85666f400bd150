"""The no-allocation backprojection against mbp_backproject, through the C ABI (GPU).

mbp_backproject_noalloc takes every device buffer from the library's 128 MiB scratch array
and allocates nothing; its results must match mbp_backproject's to the parity bar (relative
L2 <= 1e-5, max relative <= 1e-4 per voxel with a floor of 1e-6 of the largest value): both
sum the same chords, in view batches of different sizes. Two calls in a row, the second
with a smaller input, so that the second runs on what the first left in the scratch.
"""

import ctypes

import numpy as np
import pytest

from workloads import CONFIGS, SMALL_CONFIGS, config_trajectory

pytestmark = pytest.mark.gpu


def _call(lib, name, plan, sino, batch, vol, accumulate, torch):
    stream = torch.cuda.current_stream().cuda_stream
    return getattr(lib, name)(plan._handle, ctypes.c_void_p(sino.data_ptr()), batch,
                              ctypes.c_void_p(vol.data_ptr()), accumulate, ctypes.c_void_p(stream))


def _check(g, o, what):
    g = g.double().cpu().numpy().ravel()
    o = o.double().cpu().numpy().ravel()
    e2 = float(np.linalg.norm(g - o) / np.linalg.norm(o))
    em = float((np.abs(g - o) / np.maximum(np.abs(o), 1e-6 * np.abs(o).max())).max())
    print(f"  {what}: rel-L2 {e2:.2e}  max-rel {em:.2e}", flush=True)
    assert e2 <= 1e-5 and em <= 1e-4, (what, e2, em)


def _plan(mbp, cfg):
    return mbp.Plan(cfg.beam, cfg.shape, cfg.spacing, config_trajectory(cfg), (cfg.rows, cfg.cols),
                    (cfg.dv, cfg.du), layout=cfg.layout)


def test_noalloc_backprojection_matches_backproject():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import matched_backprojection_amd as mbp
    from matched_backprojection_amd import _capi
    lib = _capi.load()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(97)
    # first call: the 512^3 cone, volume z-fastest and used in place; the scratch holds about
    # 80 of its 720 views' reordered sinogram, so the gather runs in view batches
    cfg = CONFIGS["c4_cone512_aniso"]
    print(f"case no-alloc {cfg.name} B=1", flush=True)
    plan = _plan(mbp, cfg)
    y = torch.rand((cfg.views, cfg.rows, cfg.cols), generator=gen, device=dev)
    ref = plan.backproject(y)
    out = plan.empty_volume(device=dev)
    out.fill_(float("nan"))
    assert _call(lib, "mbp_backproject_noalloc", plan, y, 1, out, 0, torch) == 0, lib.mbp_last_error()
    torch.cuda.synchronize()
    info = plan.info
    print(f"  {info['last_adjoint']}, {info['last_adjoint_views_per_launch']} views per launch", flush=True)
    assert info["last_adjoint"] == "gather" and info["last_adjoint_views_per_launch"] < cfg.views
    _check(out, ref, "no-alloc vs backproject")
    plan.close()
    del y, ref, out
    # second call, smaller: the 256^3 cone's twin, (D, H, W) volumes, a batch of two (the
    # interleaved z-fastest volume also lives in the scratch), then adding into a prefilled
    # output
    cfg = SMALL_CONFIGS["c3_cone256"]
    print(f"case no-alloc {cfg.name} B=2", flush=True)
    plan = _plan(mbp, cfg)
    y = torch.rand((2, cfg.views, cfg.rows, cfg.cols), generator=gen, device=dev)
    ref = plan.backproject(y)
    out = plan.empty_volume(2, device=dev)
    out.fill_(float("nan"))
    assert _call(lib, "mbp_backproject_noalloc", plan, y, 2, out, 0, torch) == 0, lib.mbp_last_error()
    torch.cuda.synchronize()
    assert plan.info["last_adjoint"] == "gather"
    _check(out, ref, "no-alloc vs backproject, batch of two")
    pre = torch.rand(out.shape, generator=gen, device=dev)
    out.copy_(pre)
    assert _call(lib, "mbp_backproject_noalloc", plan, y, 2, out, 1, torch) == 0, lib.mbp_last_error()
    torch.cuda.synchronize()
    _check(out, ref + pre, "no-alloc accumulate")
    plan.close()
