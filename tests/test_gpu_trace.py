"""MBP_TRACE: with the variable set, every launch prints its kernel, grid, block, dynamic LDS
bytes and work range to stderr; unset, nothing is printed (GPU)."""

import os
import re

import numpy as np
import pytest

from workloads import SMALL_CONFIGS, config_phantom, config_trajectory

pytestmark = pytest.mark.gpu


def test_trace_prints_each_launch(capfd):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import matched_backprojection_amd as mbp
    cfg = SMALL_CONFIGS["c3_cone256"]
    plan = mbp.Plan("cone", cfg.shape, cfg.spacing, config_trajectory(cfg), (cfg.rows, cfg.cols),
                    (cfg.dv, cfg.du))
    x = torch.from_numpy(config_phantom(cfg)).to("cuda")
    plan.set_view_batch(20)                          # 36 views: launches of 20 and 16
    plan.set_orbit(False)                            # every view walked (see below for the half turn)
    os.environ["MBP_TRACE"] = "1"
    try:
        y = plan.project(x)
        plan.backproject(y)
        torch.cuda.synchronize()
    finally:
        del os.environ["MBP_TRACE"]
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("mbp-trace ")]
    print("\n".join(lines))
    pat = re.compile(r"^mbp-trace (\S+) grid (\d+) x (\d+) x (\d+) block (\d+) lds (\d+) ?(.*)$")
    parsed = [pat.match(l) for l in lines]
    assert all(parsed), lines
    kernels = [m.group(1) for m in parsed]
    # the (D, H, W) volume goes to the z-fastest layout, the forward runs in two view launches,
    # the adjoint's pre-pass and gather run per view batch, then back to (D, H, W)
    assert kernels.count("column_forward_kernel<flat>") == 2
    assert kernels.count("sino_prepass_kernel") == 2 and kernels.count("column_gather_kernel") == 2
    assert "dhw_to_native_kernel" in kernels and "native_to_dhw_kernel" in kernels
    fwd = [m for m in parsed if m.group(1) == "column_forward_kernel<flat>"]
    assert "views 0..19" in fwd[0].group(7) and "views 20..35" in fwd[1].group(7)
    # one block per (view, 4 adjacent columns, 64-row block), 4 waves each
    quads, row_blocks = -(-cfg.cols // 4), -(-cfg.rows // 64)
    assert [int(m.group(2)) for m in fwd] == [20 * quads * row_blocks, 16 * quads * row_blocks]
    assert all(int(m.group(5)) == 256 for m in fwd)
    gat = [m for m in parsed if m.group(1) == "column_gather_kernel"]
    assert all(int(m.group(6)) > 0 and int(m.group(5)) == 256 for m in gat)
    # the 36 views on a 56-wide grid have a half-turn symmetry: with all views in one launch,
    # the forward walks views 0..17 only (each walk also giving the view 18 later), the
    # pre-pass pairs views 18 apart and one gather serves both cells of each pair
    assert plan.info["orbit"] == 2
    plan.set_orbit(True)
    plan.set_view_batch(0)
    os.environ["MBP_TRACE"] = "1"
    try:
        y = plan.project(x)
        plan.backproject(y)
        torch.cuda.synchronize()
    finally:
        del os.environ["MBP_TRACE"]
    lines = [l for l in capfd.readouterr().err.splitlines() if l.startswith("mbp-trace ")]
    print("\n".join(lines))
    parsed = [pat.match(l) for l in lines]
    fwd = [m for m in parsed if m.group(1) == "column_forward_kernel<flat>"]
    assert len(fwd) == 1 and "views 0..17 members 1 orbit 2" in fwd[0].group(7)
    assert int(fwd[0].group(2)) == 18 * quads * row_blocks
    pre = [m for m in parsed if m.group(1) == "sino_prepass_kernel"]
    assert len(pre) == 1 and "views 0..17 members 2" in pre[0].group(7) and "apart 18" in pre[0].group(7)
    gat = [m for m in parsed if m.group(1) == "column_gather_kernel"]
    assert len(gat) == 1 and "members 1 orbit 2" in gat[0].group(7)
    assert plan.info["last_forward_orbit"] == 2 and plan.info["last_adjoint_orbit"] == 2
    # unset: silent
    plan.project(x)
    torch.cuda.synchronize()
    assert "mbp-trace" not in capfd.readouterr().err
    plan.close()
