"""Throughput of the cone-beam forward + matched backprojection pair on one MI355X.

Workload: the 512^3 anisotropic circular cone beam (volume stored z-fastest, spacing
(dz, dy, dx) = (1.5, 1, 1), SID 1000, SDD 1500, 720 views, 768 x 512 detector, 20 seeded
ellipsoids plus U[0, 0.05) background). One step = one forward projection of the phantom and
one matched backprojection of the resulting sinogram (every row of the hot path: frame
staging is done once per plan, ray setup, forward walk, adjoint walk; this workload needs no
layout conversion and fits one view launch).

Metric: ray/voxel segments of positive length walked per second, forward plus adjoint,
divided by the time of both (G ray-segments/s). The segment count comes from the library's
counting kernel. Timing: W untimed warm-up steps, then K timed steps between device
synchronisations; per-operation kernel time from HIP events recorded on the stream the
kernels run on.

Printed: one JSON line with the metric, a roofline object for the dominant kernel
(algorithmic bytes per launch / average launch time, against the 8 TB/s HBM peak) and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c4_cone512_hbm_traffic.md")


def kernel_source_hash() -> str:
    """sha256 over the kernel sources (the key the traffic measurements are stored under)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("kernels.hip", "traverse.h", "mbp_internal.h"):
        with open(os.path.join(ROOT, "matched_backprojection_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            line = next(l for l in f if l.startswith("traffic-json:"))
    except (OSError, StopIteration):
        return None
    rec = json.loads(line.split(":", 1)[1])
    if rec.get("source_sha256") != kernel_source_hash() or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return float(k["read_bytes"] + k["write_bytes"])


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(cfg, traj, x_dhw, views=(0, 180, 360, 540)):
    """The fp64 oracle on all rays of a few views: forward, then adjoint of its output."""
    import numpy as np
    from oracle import oracle as O

    geom = O.geom_from_config(cfg)
    sub = {k: (None if v is None else np.ascontiguousarray(v[list(views)])) for k, v in traj.items()}
    sgeom = dict(geom, views=len(views))
    threads = O.max_threads()
    t0 = time.perf_counter()
    sino, counts = O.project(sgeom, sub, x_dhw, counts=True)
    t1 = time.perf_counter()
    O.backproject(sgeom, sub, sino.astype(np.float32))
    t2 = time.perf_counter()
    segs = int(counts.sum())
    value = 2 * segs / (t2 - t0) / 1e9
    log(f"cpu oracle: {segs} segments per op, forward {t1 - t0:.2f} s, adjoint {t2 - t1:.2f} s, "
        f"{threads} threads")
    return {"value": value, "unit": "Gray-segments/s", "cores": threads, "kind": "oracle",
            "sample": (f"views {list(views)} of {cfg.views} (all {cfg.rows}x{cfg.cols} rays each), "
                       f"fp64 forward then adjoint; {segs} segments per op; "
                       f"{t2 - t0:.1f} s total")}


def measure_pair(mbp, torch, cfg, steps: int, warmup: int) -> dict:
    """Forward + matched backprojection of one configuration (its own layout and batch), timed
    like the headline pair; for the secondary workloads reported next to it."""
    import numpy as np
    from workloads import config_phantom, config_trajectory
    dev = torch.device("cuda:0")
    traj = config_trajectory(cfg)
    x = config_phantom(cfg)
    plan = mbp.Plan(cfg.beam, cfg.shape, cfg.spacing, traj, (cfg.rows, cfg.cols), (cfg.dv, cfg.du),
                    layout=cfg.layout)
    batch = cfg.batch or None
    xs = x if batch else x[None]
    if cfg.layout == "WHD":
        xd = torch.from_numpy(np.ascontiguousarray(xs.transpose(0, 3, 2, 1))).to(dev).permute(0, 3, 2, 1)
    else:
        xd = torch.from_numpy(np.ascontiguousarray(xs)).to(dev)
    if not batch:
        xd = xd[0]
    sino = torch.empty(((batch,) if batch else ()) + plan.sino_shape, dtype=torch.float32, device=dev)
    vol = plan.empty_volume(batch, device=dev)
    segs = plan.segment_count() * (batch or 1)
    for _ in range(warmup):
        plan.project(xd, out=sino)
        plan.backproject(sino, out=vol)
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        plan.project(xd, out=sino)
        ev[1].record()
        plan.backproject(sino, out=vol)
        ev[2].record()
        events.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    io = 4.0 * (cfg.n_voxels + cfg.n_rays) * (batch or 1) + 96.0 * cfg.views
    alg = 4.0 * segs + io
    out = {"workload": cfg.name, "batch": cfg.batch, "layout": cfg.layout, "path": plan.info["path"],
           "segments_per_op": segs, "forward_ms": f_ms, "adjoint_ms": b_ms,
           "gsegments_per_s": 2.0 * segs * steps / wall / 1e9,
           "rays_per_s": 2.0 * cfg.n_rays * (batch or 1) * steps / wall,
           "pct_hbm_peak_pair": 100.0 * 2 * alg / ((f_ms + b_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS}
    log(f"{cfg.name}: forward {f_ms:.2f} ms, adjoint {b_ms:.2f} ms, "
        f"{out['gsegments_per_s']:.0f} G segments/s, {out['pct_hbm_peak_pair']:.1f}% of HBM peak")
    plan.close()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--adjoint", choices=("gather", "scatter"), default="gather",
                    help="adjoint kernel of the column walk")
    ap.add_argument("--cgls", type=int, default=10,
                    help="iterations of the CGLS solve timed for context (0: skip)")
    ap.add_argument("--no-others", dest="others", action="store_false",
                    help="skip timing the 256^3 cone, the batched helical cone and the tilted cone")
    ap.add_argument("--probe", action="store_true",
                    help="for hardware-counter runs: one forward, one adjoint and a 1 GiB "
                         "device-to-device copy (the counters' calibration), no timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is "
              "a design, not part of this build", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import matched_backprojection_amd as mbp
    from workloads import CONFIGS, config_phantom, config_trajectory

    cfg = CONFIGS["c4_cone512_aniso"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = time.perf_counter()
    traj = config_trajectory(cfg)
    x = config_phantom(cfg)
    log(f"phantom {cfg.shape} built in {time.perf_counter() - t:.1f} s")
    plan = mbp.Plan("cone", cfg.shape, cfg.spacing, traj, (cfg.rows, cfg.cols), (cfg.dv, cfg.du),
                    layout="WHD")
    plan.set_adjoint(args.adjoint)
    info = plan.info
    # the z-fastest volume: a (D, H, W) tensor with strides (1, D, D*H)
    xd = torch.from_numpy(np.ascontiguousarray(x.transpose(2, 1, 0))).to(dev).permute(2, 1, 0)
    sino = torch.empty((cfg.views, cfg.rows, cfg.cols), dtype=torch.float32, device=dev)
    vol = plan.empty_volume(device=dev)
    if args.probe:
        plan.project(xd, out=sino)
        plan.backproject(sino, out=vol)
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)                        # 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        log("probe: forward, adjoint and a 1 GiB copy done")
        plan.close()
        return 0
    segs = plan.segment_count()
    log(f"plan: {info}; {segs} positive-length segments per op")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        plan.project(xd, out=sino)
        if ev is not None:
            ev[1].record()
        plan.backproject(sino, out=vol)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    value = 2.0 * segs * args.steps / wall / 1e9
    f_avg, b_avg = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    log(f"forward {f_avg:.2f} ms (median {np.median(fwd_ms):.2f}), adjoint {b_avg:.2f} ms "
        f"(median {np.median(bwd_ms):.2f}), step {ms_per_step:.2f} ms wall")

    io_bytes = 4.0 * (cfg.n_voxels + cfg.n_rays) + 96.0 * cfg.views
    alg_bytes = 4.0 * segs + io_bytes
    adj_kernel = "column_gather_kernel" if args.adjoint == "gather" else "column_adjoint_kernel"
    dominant = adj_kernel if b_avg >= f_avg else "column_forward_kernel"
    dom_ms = max(b_avg, f_avg)
    achieved = alg_bytes / (dom_ms * 1e-3) / 1e9
    traffic = measured_traffic(dominant)
    pair_gbs = 2 * alg_bytes / ((f_avg + b_avg) * 1e-3) / 1e9
    log(f"algorithmic bytes per launch {alg_bytes / 1e9:.1f} GB; dominant {dominant}: "
        f"{achieved:.0f} GB/s = {achieved / HBM_PEAK_GBS:.3f} of peak; pair {pair_gbs:.0f} GB/s")

    result = {
        "metric": "cone forward+backproject Gray-segments/s at 512^3 on 1 MI355X; % HBM peak",
        "value": value,
        "unit": "Gray-segments/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("c4_cone512_aniso: circular cone beam, 512^3 volume stored "
                         "(W,H,D)-contiguous, spacing (dz,dy,dx)=(1.5,1,1), SID 1000, SDD 1500, "
                         "720 views, 768 cols x 512 rows, pitch 1; 20 seeded ellipsoids + "
                         "U[0,0.05) background; forward + matched backprojection"),
            "segments_per_op": segs,
            "rays_per_op": cfg.n_rays,
            "path": info["path"],
            "adjoint_kernel": adj_kernel,
            "forward_ms": f_avg,
            "adjoint_ms": b_avg,
            "rays_per_s": 2.0 * cfg.n_rays * args.steps / wall,
            "pct_hbm_peak_pair": 100.0 * pair_gbs / HBM_PEAK_GBS,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dominant,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
    }
    # context: the HBM bandwidth a plain device-to-device copy reaches on this GPU (2 GiB read
    # and 2 GiB written per copy), and each kernel's algorithmic rate against it
    src = torch.empty(1 << 29, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = []
    for _ in range(5):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        copy_ms.append(ev[0].elapsed_time(ev[1]))
    copy_gbs = 2.0 * src.numel() * 4 / (float(np.median(copy_ms)) * 1e-3) / 1e9
    del src, dst
    log(f"device-to-device copy: {copy_gbs:.0f} GB/s")
    result["config"]["hbm_copy_GBs"] = copy_gbs
    result["config"]["forward_GBs_algorithmic"] = alg_bytes / (f_avg * 1e-3) / 1e9
    result["config"]["adjoint_GBs_algorithmic"] = alg_bytes / (b_avg * 1e-3) / 1e9
    result["config"]["pct_copy_bandwidth_pair"] = 100.0 * pair_gbs / copy_gbs
    if args.cgls > 0:
        # context, not the headline: one CGLS solve of args.cgls iterations on the same
        # workload after a two-iteration warm-up solve (the pages time ten-iteration solves
        # and divide by ten), volumes kept z-fastest, sinogram = the forward projection above
        ws = torch.empty(plan.cgls_workspace_size(1, args.cgls), dtype=torch.uint8, device=dev)
        xc = plan.empty_volume(device=dev)
        xc.zero_()
        plan.cgls(sino, 2, x0=xc, workspace=ws)
        xc.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, hist = plan.cgls(sino, args.cgls, x0=xc, workspace=ws)
        torch.cuda.synchronize()
        cg_ms = (time.perf_counter() - t0) * 1e3 / args.cgls
        log(f"CGLS: {args.cgls} iterations, {cg_ms:.1f} ms per iteration (including the start), "
            f"residual {hist[0]:.4g} -> {hist[-1]:.4g}")
        result["config"]["cgls_iter_ms"] = cg_ms
        result["config"]["cgls_iters"] = args.cgls
        del ws, xc
    if args.others:
        # the 256^3 cone of the metric, the batched helical cone, and the 256^3 cone with its
        # detector tilted by a few degrees in its plane (rows no longer along z: the generic
        # walk with the atomic adjoint), volume z-fastest; timed the same way
        from dataclasses import replace
        tilted = replace(CONFIGS["c3_cone256"], name="c3_cone256_tilted",
                         trajectory="circular_tilted", layout="WHD")
        result["config"]["other_workloads"] = [
            measure_pair(mbp, torch, c, steps=5, warmup=2)
            for c in (CONFIGS["c3_cone256"], CONFIGS["c5_helical_b4"], tilted)]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, traj, x)
    print(json.dumps(result), flush=True)
    plan.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
