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
synchronisations (defaults 3 and 7: the pages time the median of seven samples after three
warm-ups, "diffct 2.1.0 -> 2.2.1", README performance section); per-operation times from HIP
events recorded on the stream the kernels run on, reported as means and medians.

Printed: one JSON line with the metric, a roofline object for the dominant kernel
(algorithmic bytes per launch / average launch time, against the 8 TB/s HBM peak, with the
bytes the kernel really moves and its instruction issue from hardware counters when those
were taken on the current sources) and the fp64 CPU oracle timed on a bounded sample of the
same workload.
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
# MI355X: 256 compute units of 4 SIMDs at 2.4 GHz; a wave64 instruction on 32-bit operands
# occupies its SIMD for 2 cycles (fp64 for 4), so one SIMD issues at most one such VALU
# instruction every 2 cycles
CUS, SIMDS_PER_CU, CLOCK_HZ, VALU_CYCLES = 256, 4, 2.4e9, 2.0
VALU_PEAK_PER_S = CUS * SIMDS_PER_CU * CLOCK_HZ / VALU_CYCLES
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c4_cone512_hbm_traffic.md")
SQ_FILE = os.path.join(ROOT, "profiles", "c4_cone512_sq_counters.md")


def kernel_source_hash() -> str:
    """sha256 over the kernel sources (the key the traffic measurements are stored under)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("kernels.hip", "traverse.h", "mbp_internal.h"):
        with open(os.path.join(ROOT, "matched_backprojection_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_record(path: str, tag: str, kernel: str):
    """Per-launch counter values of `kernel` from the machine-readable line `tag` of a
    committed counter summary, or None when the kernel sources changed since the counters
    were taken (or there is no such record)."""
    try:
        with open(path) as f:
            line = next(l for l in f if l.startswith(tag + ":"))
    except (OSError, StopIteration):
        return None
    rec = json.loads(line.split(":", 1)[1])
    if rec.get("source_sha256") != kernel_source_hash() or kernel not in rec.get("kernels", {}):
        return None
    return rec["kernels"][kernel]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE), or None."""
    k = counter_record(TRAFFIC_FILE, "traffic-json", kernel)
    return None if k is None else float(k["read_bytes"] + k["write_bytes"])


def issue_record(kernel: str, segments: int, kernel_ms: float):
    """Instruction issue of `kernel` from its SQ counters: VALU instructions per segment, the
    issue rate they give over the live launch time against one wave64 32-bit VALU
    instruction per 2 cycles per SIMD, the counters' own VALU-busy share of SIMD cycles and
    LDS-busy share of CU cycles; None without counters for the current sources."""
    k = counter_record(SQ_FILE, "sq-json", kernel)
    if k is None:
        return None
    valu = float(k["SQ_INSTS_VALU"])
    rate = valu / (kernel_ms * 1e-3)
    out = {"valu_insts_per_segment": valu / segments,
           "salu_insts_per_segment": float(k["SQ_INSTS_SALU"]) / segments,
           "lds_insts_per_segment": float(k["SQ_INSTS_LDS"]) / segments,
           "achieved": rate, "peak": VALU_PEAK_PER_S, "unit": "wave64 VALU instructions/s",
           "frac": rate / VALU_PEAK_PER_S, "valu_busy": float(k["valu_busy"])}
    if "fp64_insts" in k:
        out["fp64_share_of_valu"] = float(k["fp64_insts"]) / valu
    if "lds_busy" in k:
        out["lds_busy"] = float(k["lds_busy"])
    return out


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, traj, x_dhw, every: int = 12):
    """The fp64 oracle on all rays of every `every`-th view: the forward, then the adjoint of
    its output, each timed on its own; the value is the pair rate, like the headline's."""
    import numpy as np
    from oracle import oracle as O

    views = list(range(0, cfg.views, every))
    geom = O.geom_from_config(cfg)
    sub = {k: (None if v is None else np.ascontiguousarray(v[views])) for k, v in traj.items()}
    sgeom = dict(geom, views=len(views))
    threads = O.max_threads()
    t0 = time.perf_counter()
    sino, counts = O.project(sgeom, sub, x_dhw, counts=True)
    t1 = time.perf_counter()
    O.backproject(sgeom, sub, sino.astype(np.float32))
    t2 = time.perf_counter()
    segs = int(counts.sum())
    model = cpu_model()
    log(f"cpu oracle ({model}, {threads} threads): {len(views)} views, {segs} segments per op, "
        f"forward {t1 - t0:.1f} s, adjoint {t2 - t1:.1f} s")
    return {"value": 2 * segs / (t2 - t0) / 1e9, "unit": "Gray-segments/s", "cores": threads,
            "kind": "oracle", "cpu_model": model,
            "forward_Gsegments_per_s": segs / (t1 - t0) / 1e9,
            "adjoint_Gsegments_per_s": segs / (t2 - t1) / 1e9,
            "forward_s": t1 - t0, "adjoint_s": t2 - t1,
            "sample": (f"every {every}th view ({len(views)} of {cfg.views}, all {cfg.rows}x{cfg.cols} "
                       f"rays each) of the headline workload; fp64 forward, then the adjoint of its "
                       f"output (per-thread fp64 volumes reduced in a fixed order); {segs} segments "
                       f"per op; {t2 - t0:.1f} s total on {threads} threads")}


def time_ops(torch, fwd, bwd, steps: int, warmup: int):
    """Warm-up steps, then `steps` timed steps of fwd() then bwd(): per-op HIP event times
    (ms) and the wall time of all timed steps (s)."""
    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for ev in events:
        ev[0].record()
        fwd()
        ev[1].record()
        bwd()
        ev[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = [e[0].elapsed_time(e[1]) for e in events]
    b_ms = [e[1].elapsed_time(e[2]) for e in events]
    return f_ms, b_ms, wall


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
    f_all, b_all, wall = time_ops(torch, lambda: plan.project(xd, out=sino),
                                  lambda: plan.backproject(sino, out=vol), steps, warmup)
    f_ms, b_ms = float(np.mean(f_all)), float(np.mean(b_all))
    io = 4.0 * (cfg.n_voxels + cfg.n_rays) * (batch or 1) + 96.0 * cfg.views
    alg = 4.0 * segs + io
    out = {"workload": cfg.name, "batch": cfg.batch, "layout": cfg.layout, "path": plan.info["path"],
           "segments_per_op": segs, "forward_ms": f_ms, "adjoint_ms": b_ms,
           "forward_ms_median": float(np.median(f_all)), "adjoint_ms_median": float(np.median(b_all)),
           "gsegments_per_s": 2.0 * segs * steps / wall / 1e9,
           "rays_per_s": 2.0 * cfg.n_rays * (batch or 1) * steps / wall,
           "pct_hbm_peak_pair": 100.0 * 2 * alg / ((f_ms + b_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS}
    log(f"{cfg.name}: forward {f_ms:.2f} ms, adjoint {b_ms:.2f} ms, "
        f"{out['gsegments_per_s']:.0f} G segments/s, {out['pct_hbm_peak_pair']:.1f}% of HBM peak")
    plan.close()
    return out


PROBE_WORKLOADS = ("c4_cone512_aniso", "c3_cone256", "c5_helical_b4", "c3_cone256_tilted",
                   "pages_cone512_360v")


def workload(name: str):
    """A configuration by name: the five configurations, the pages' context workload, and
    the 256^3 cone with its detector rotated in its plane (volume z-fastest)."""
    from dataclasses import replace
    from workloads import CONFIGS
    from workloads.configs import CONTEXT_CONFIGS
    if name == "c3_cone256_tilted":
        return replace(CONFIGS["c3_cone256"], name=name, trajectory="circular_tilted", layout="WHD")
    return CONFIGS.get(name) or CONTEXT_CONFIGS[name]


def probe(mbp, torch, name: str) -> int:
    """For hardware-counter runs: one forward and one adjoint of workload `name`, then a 1 GiB
    streaming copy (1 GiB read + 1 GiB written: the counters' calibration); no timing."""
    import numpy as np
    from workloads import config_phantom, config_trajectory
    cfg = workload(name)
    dev = torch.device("cuda:0")
    plan = mbp.Plan(cfg.beam, cfg.shape, cfg.spacing, config_trajectory(cfg), (cfg.rows, cfg.cols),
                    (cfg.dv, cfg.du), layout=cfg.layout)
    x = config_phantom(cfg)
    xs = x if cfg.batch else x[None]
    if cfg.layout == "WHD":
        xd = torch.from_numpy(np.ascontiguousarray(xs.transpose(0, 3, 2, 1))).to(dev).permute(0, 3, 2, 1)
    else:
        xd = torch.from_numpy(np.ascontiguousarray(xs)).to(dev)
    if not cfg.batch:
        xd = xd[0]
    sino = plan.project(xd)
    plan.backproject(sino)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    mbp.stream_copy(src, dst)
    torch.cuda.synchronize()
    log(f"probe {name}: forward, adjoint and a 1 GiB streaming copy done")
    plan.close()
    return 0


def copy_bandwidth(mbp, torch, dev) -> float:
    """HBM rate of the library's streaming copy, 2 GiB read + 2 GiB written, median of 5."""
    import numpy as np
    src = torch.empty(1 << 29, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    mbp.stream_copy(src, dst)
    ms = []
    for _ in range(5):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        mbp.stream_copy(src, dst)
        ev[1].record()
        torch.cuda.synchronize()
        ms.append(ev[0].elapsed_time(ev[1]))
    del src, dst
    return 2.0 * (1 << 29) * 4 / (float(np.median(ms)) * 1e-3) / 1e9


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=7)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-every", type=int, default=12,
                    help="the CPU oracle baseline runs every n-th view of the headline workload")
    ap.add_argument("--adjoint", choices=("gather", "scatter"), default="gather",
                    help="adjoint kernel of the column walk")
    ap.add_argument("--cgls", type=int, default=10,
                    help="iterations of the CGLS solve timed for context (0: skip)")
    ap.add_argument("--no-others", dest="others", action="store_false",
                    help="skip timing the other workloads (256^3 cone, batched helical cone, "
                         "tilted cone, the pages' 360-view cone)")
    ap.add_argument("--probe", nargs="?", const="c4_cone512_aniso", default=None,
                    choices=PROBE_WORKLOADS,
                    help="for hardware-counter runs: one forward, one adjoint of the workload and "
                         "a 1 GiB streaming copy (the counters' calibration), no timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is "
              "a design, not part of this build", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import matched_backprojection_amd as mbp
    from workloads import CONFIGS, config_phantom, config_trajectory

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.probe:
        return probe(mbp, torch, args.probe)
    cfg = CONFIGS["c4_cone512_aniso"]
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
    segs = plan.segment_count()
    log(f"plan: {info}; {segs} positive-length segments per op")

    fwd_ms, bwd_ms, wall = time_ops(torch, lambda: plan.project(xd, out=sino),
                                    lambda: plan.backproject(sino, out=vol), args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    value = 2.0 * segs * args.steps / wall / 1e9
    f_avg, b_avg = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    f_med, b_med = float(np.median(fwd_ms)), float(np.median(bwd_ms))
    log(f"forward {f_avg:.2f} ms (median {f_med:.2f}), adjoint {b_avg:.2f} ms "
        f"(median {b_med:.2f}), step {ms_per_step:.2f} ms wall")

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
    roof = {
        "bound": "hbm",
        "kernel": dominant,
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": traffic,
        "note": ("achieved = algorithmic bytes (4 B per segment + compulsory I/O) / launch time, "
                 "a normalised segment rate; traffic = the bytes the kernel moves to and from "
                 "memory (calibrated counters), traffic_GBs its rate; issue = its VALU issue "
                 "from SQ counters"),
    }
    if traffic is not None:
        roof["traffic_GBs"] = traffic / (dom_ms * 1e-3) / 1e9
        roof["traffic_frac"] = roof["traffic_GBs"] / HBM_PEAK_GBS
    issue = issue_record(dominant, segs, dom_ms)
    if issue is not None:
        roof["issue"] = issue
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
            "forward_ms_median": f_med,
            "adjoint_ms_median": b_med,
            "rays_per_s": 2.0 * cfg.n_rays * args.steps / wall,
            "pct_hbm_peak_pair": 100.0 * pair_gbs / HBM_PEAK_GBS,
        },
        "roofline": roof,
    }
    for k in ("forward", "adjoint"):
        kern = "column_forward_kernel" if k == "forward" else adj_kernel
        ms = f_avg if k == "forward" else b_avg
        result["config"][f"{k}_GBs_algorithmic"] = alg_bytes / (ms * 1e-3) / 1e9
        tr = measured_traffic(kern)
        if tr is not None:
            result["config"][f"{k}_GBs_traffic"] = tr / (ms * 1e-3) / 1e9
        iss = issue_record(kern, segs, ms)
        if iss is not None:
            result["config"][f"{k}_valu_insts_per_segment"] = iss["valu_insts_per_segment"]
            result["config"][f"{k}_valu_busy"] = iss["valu_busy"]
            if "lds_busy" in iss:
                result["config"][f"{k}_lds_busy"] = iss["lds_busy"]
    copy_gbs = copy_bandwidth(mbp, torch, dev)
    log(f"streaming copy: {copy_gbs:.0f} GB/s")
    result["config"]["hbm_copy_GBs"] = copy_gbs
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
        # the 256^3 cone of the metric, the batched helical cone, the 256^3 cone with its
        # detector tilted by a few degrees in its plane (rows no longer along z: the generic
        # walk forward and the per-row gather), and the pages' own 512^3 workload (360 views,
        # 1024 x 768 at pitch 1.25), each timed like the headline pair
        result["config"]["other_workloads"] = [
            measure_pair(mbp, torch, workload(n), steps=5, warmup=2)
            for n in ("c3_cone256", "c5_helical_b4", "c3_cone256_tilted", "pages_cone512_360v")]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, traj, x, every=args.cpu_every)
    print(json.dumps(result), flush=True)
    plan.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
