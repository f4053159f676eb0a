"""Benchmark: one training step (preprocess, keys, sort, ranges, forward
raster, L1 loss, backward raster, preprocess backward, Adam) of the tile-based
differentiable Gaussian rasterizer on one MI355X.

Workload: 1M Gaussians, SH degree 3, a batch of 4 views at 1920x1080 (yaw
0/5/10/15 degrees about the scene centre), L1 against the render of a second
seeded scene, fp32. Inputs are synthetic and resident in HBM before timing.

Prints one JSON line. `value` is iterations/s of the whole step; Mpix/s and
the per-stage breakdown ride along. The roofline object describes the step's
dominant kernel, timed with HIP events on the stream it runs on: for a raster
kernel, fp32 work is 12 flops per evaluated (pixel, entry) pair -- every entry
of a pixel's list up to its last contributor, summed from n_contrib -- against
the fp32 FMA rate without packed math; for the others, algorithmic HBM bytes
against 8 TB/s. `traffic` is the kernel's measured HBM bytes per dispatch from
the committed counter summary (null once the kernel's sources have changed).
The cpu_baseline object times the CPU oracle on a bounded sample on this host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
# fp32 FMA rate without packed-fp32 instructions (which this build leaves
# disabled): 256 CUs x 64 lanes x 2 flops x 2.4 GHz. The published 157.3
# TFLOP/s counts packed (two-wide) fp32.
FP32_FMA_PEAK_TFLOPS = 78.6
# fp32 operations every evaluated (pixel, entry) pair costs in either raster
# pass: dx, dy (2), the power polynomial (3 mul + 2 fma = 7), exp (1),
# opacity x G (1), the 0.99 clamp (1)
FLOPS_PER_PAIR = 12
METRIC = "fwd+bwd+Adam iters/s & Mpix/s, 1M Gaussians SH3 @1080p; % of HBM roofline"
CSRC = os.path.join(ROOT, "gaussian_splatting_differentiable_ewa_amd", "csrc")
# sources each kernel is built from (a change voids its stored traffic counts)
KERNEL_SOURCES = {
    "k_raster_bwd": ["raster_bwd.hip", "raster_bwd.h", "raster_common.h", "internal.h", "common.h"],
    "k_raster_fwd": ["raster_fwd.hip", "raster_fwd.h", "raster_common.h", "internal.h", "common.h"],
    "k_raster_fwd_l1": ["raster_fwd.hip", "raster_fwd.h", "raster_common.h", "internal.h", "common.h"],
    "k_raster_fwd_bwd_l1": ["raster_fused.hip", "raster_fwd.h", "raster_bwd.h", "raster_common.h", "internal.h",
                            "common.h"],
    "k_adam": ["optim.hip", "adam.h", "internal.h", "common.h"],
    "k_preprocess_bwd": ["preprocess_bwd.hip", "adam.h", "project.h", "internal.h", "common.h"],
    "k_tile_masks": ["tile_masks.hip", "raster_common.h", "internal.h", "common.h"],
}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(PROFILES, f"traffic_{workload}.md")


def stored_traffic(workload, kernel):
    """HBM bytes per dispatch of `kernel` from the committed counter summary,
    or None when there is none or the kernel's sources changed since."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    digest = kernel_digest(kernel)
    with open(path) as fh:
        for line in fh:
            parts = line.strip().strip("|").split("|")
            parts = [p.strip() for p in parts]
            if len(parts) >= 6 and parts[0] == kernel and parts[5] == digest:
                try:
                    return int(parts[4])
                except ValueError:
                    return None
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="scene id (2 = the headline workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lists", choices=["auto", "binned", "radix"], default="auto",
                    help="list builder: binning per tile, the global key sort, or chosen per scene")
    ap.add_argument("--no-state-flags", action="store_true",
                    help="dense Adam: read every Gaussian's moments, also those known to be zero and unseen")
    ap.add_argument("--generated-order", action="store_true",
                    help="keep the Gaussians in the generated (random) order instead of the Morton order of their means")
    ap.add_argument("--separate-raster", action="store_true",
                    help="forward + loss and backward raster as two passes instead of the fused one")
    ap.add_argument("--band-rows", type=int, default=None,
                    help="memory-capped mode: lists and raster one window of this many tile rows at a time")
    ap.add_argument("--cpu-sample-views", type=int, default=1,
                    help="views of the workload the CPU oracle runs (its time is scaled to all views)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no benchmark: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, csv output) into the traffic summary under profiles/")
    ap.add_argument("--traffic-command", default="",
                    help="the counter command, COUNTER standing for the counter name (quoted in the summary)")
    return ap.parse_args()


def stage_bytes(P, n, V, K, n_vis_per_view, n_any, n_px, n_adam=None):
    """Algorithmic HBM bytes per stage of one step (what the method must
    move with this layout: each input read once, each output written once).
    n_adam: the Gaussians the fused backward + Adam must read and update (all
    n, unless the per-Gaussian state flags mark some with zero moments and
    no gradient, whose update is the identity and moves nothing)."""
    n_adam = n if n_adam is None else n_adam
    Bp = 4 * P
    Nv = sum(n_vis_per_view)
    return {
        # means for culling, the rest for Gaussians visible anywhere; per view
        # a 48-byte record + 8-byte rectangle for visible pairs, a count for all
        "preprocess": 12 * n + (Bp - 12) * n_any + 56 * Nv + 4 * V * n,
        "scan": 8 * V * n,
        "emit": 16 * V * n + 12 * K,          # rect + offset per pair, key + id per intersection
        "sort": 24 * K,                       # one read + one write of key + id
        "ranges": 8 * K + 8 * V * n_px // 256,
        # per list entry: id read, record gathered, 16-bit sub-block mask written
        "tile_masks": (4 + 48 + 2) * K,
        # forward raster with the L1 loss fused: ids and masks, one record read
        # per visible pair, target read, T_final + n_contrib + dL/dimage written
        "raster_fwd_loss": 6 * K + 36 * Nv + 32 * V * n_px,
        "raster_bwd": 6 * K + 36 * Nv + 32 * V * n_px + 36 * Nv * 2,
        # the two raster passes and the loss in one: ids and masks, one record
        # read per visible pair, target read, 2D gradients zeroed and written
        "raster_fwd_bwd": 6 * K + 36 * Nv + 12 * V * n_px + 36 * Nv * 2,
        "preprocess_bwd": Bp * n_any + 44 * Nv + Bp * n,
        "adam": 7 * Bp * n,
        # the two above in one pass: every (view, Gaussian) rectangle and
        # each visible pair's 2D gradient read, the gradient never stored;
        # for each Gaussian updated, parameters and moments read once,
        # parameters and moments written
        "preprocess_bwd_adam": 8 * V * n + 36 * Nv + 6 * Bp * n_adam,
    }


def main():
    args = parse()
    if args.traffic_summary:
        from gaussian_splatting_differentiable_ewa_amd import scenes as S
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1], S.CONFIGS[args.config].name,
                        args.traffic_command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout is a design "
              "note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from gaussian_splatting_differentiable_ewa_amd import _lib as L
    from gaussian_splatting_differentiable_ewa_amd import scenes as S
    from gaussian_splatting_differentiable_ewa_amd.step import TrainStep, render, spatial_order

    L.lib()
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[args.config]
    cams = cfg.cameras()
    t0 = time.time()
    params_np = S.make_params(cfg)
    # storage order of the Gaussians: Morton order of the means (set-up, not
    # timed; the step's arithmetic does not depend on it), or as generated
    perm = None if args.generated_order else spatial_order(params_np[:3])
    params = torch.from_numpy(params_np if perm is None else np.ascontiguousarray(params_np[:, perm])).to(dev)
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    ts = TrainStep(params.clone(), cfg.sh_degree, cams, target, lr=cfg.lr, betas=(cfg.beta1, cfg.beta2),
                   eps=cfg.eps, band_rows=args.band_rows, fused_raster=not args.separate_raster, lists=args.lists,
                   state_flags=not args.no_state_flags)
    print(f"[bench] {cfg.name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    b = ts.buf
    names = ts.stage_names

    for _ in range(args.warmup):
        ts.step()
    ts.flush()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t0_applied, redone0 = ts.t, ts.redone
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        ts.step(marks=events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ts.flush()  # settles the copied counts (no GPU work left)
    applied = ts.t - t0_applied
    redone = ts.redone - redone0
    stage_ms = {nm: float(np.mean([events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps)]))
                for i, nm in enumerate(names)}
    # a step redone after a list overflow is not an update: count applied ones
    ms_per_step = wall * 1e3 / max(1, applied)
    it_s = 1e3 / ms_per_step
    V, H, W = b.V, b.H, b.W
    mpix = V * H * W * it_s / 1e6

    rect = b.rect.view(V, b.n, 4).cpu().numpy().view(np.uint16).astype(np.int32)
    vis = (rect[..., 2] > rect[..., 0]) & (rect[..., 3] > rect[..., 1])
    n_vis = [int(x) for x in vis.sum(axis=1)]
    n_any = int(vis.any(axis=0).sum())
    # with the state flags on, the fused backward + Adam touches only the
    # Gaussians whose moments are not known to be zero (those seen so far)
    n_adam = int((ts.adam_state != 0).sum()) if ts.fused_adam and ts._use_state else b.n
    sb = stage_bytes(b.P, b.n, V, b.K, n_vis, n_any, H * W, n_adam)
    unused = ["preprocess_bwd", "adam"] if ts.fused_adam else ["preprocess_bwd_adam"]
    unused += ["raster_fwd_loss", "raster_bwd"] if ts.fused_raster else ["raster_fwd_bwd"]
    step_bytes = sum(v for k, v in sb.items() if k not in unused)
    frac_step = step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9)

    # dominant kernel: the single-kernel stage with the largest time
    pairs = ts.evaluated_pairs()  # (pixel, entry) pairs up to each last contributor (after the timed steps)
    single = {"raster_fwd_loss": "k_raster_fwd_l1", "raster_bwd": "k_raster_bwd", "adam": "k_adam",
              "preprocess_bwd": "k_preprocess_bwd", "preprocess_bwd_adam": "k_preprocess_bwd",
              "raster_fwd_bwd": "k_raster_fwd_bwd_l1"}
    single = {k: v for k, v in single.items() if k in stage_ms}
    dom = max(single, key=lambda k: stage_ms[k])
    kern = single[dom]
    dur_s = stage_ms[dom] * 1e-3
    if dom.startswith("raster"):
        # the fused pass evaluates every pair twice (forward, then backward)
        per_pair = FLOPS_PER_PAIR * (2 if dom == "raster_fwd_bwd" else 1)
        flops = per_pair * pairs
        achieved = flops / dur_s / 1e12
        roofline = {"bound": "alu", "kernel": kern, "achieved": round(achieved, 3), "peak": FP32_FMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP32_FMA_PEAK_TFLOPS, 4),
                    "traffic": stored_traffic(cfg.name, kern), "algorithmic_flops": flops,
                    "pairs": pairs, "flops_per_pair": per_pair, "algorithmic_bytes": int(sb[dom]),
                    "hbm_gbs_algorithmic": round(sb[dom] / dur_s / 1e9, 1)}
    else:
        achieved = sb[dom] / dur_s / 1e9
        roofline = {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": stored_traffic(cfg.name, kern), "algorithmic_bytes": int(sb[dom])}
    roofline["avg_launch_ms"] = round(stage_ms[dom], 4)

    # intersection statistics and a plain device copy for the achievable HBM rate
    # the ranges of the lists built last: in the memory-capped mode only the
    # last window's tiles (the rest of the buffer is not theirs)
    n_rng = b.V * b.TX * (b.TY - (b.TY - 1) // args.band_rows * args.band_rows) if args.band_rows else b.V * b.T
    rng_ = b.ranges.view(-1, 2)[:n_rng].to(torch.int64)
    max_per_tile = int((rng_[:, 1] - rng_[:, 0]).max())
    peak_list_bytes = b.workspace_bytes()
    copy_gbs = copy_probe(torch, dev)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, params_np, cams, args.cpu_sample_views)

    out = {
        "metric": METRIC, "value": round(it_s, 3), "unit": "iter/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "gaussians": cfg.n, "sh_degree": cfg.sh_degree, "views": V,
                   "width": W, "height": H},
        "mpix_per_s": round(mpix, 2),
        "step_hbm_fraction": round(frac_step, 4), "step_algorithmic_bytes": int(step_bytes),
        "intersections": b.K, "k_per_gaussian": round(b.K / b.n, 4), "list_builder": b.path,
        "band_rows": args.band_rows, "raster": "separate" if args.separate_raster else "fused",
        "gaussian_order": "generated" if args.generated_order else "morton",
        "adam_state_flags": bool(ts._use_state),
        "host_count_read": not ts.defer_count or not b.lists_without_count(), "redone_steps": redone,
        "visible_per_view": n_vis, "adam_gaussians": n_adam,
        "max_per_tile": max_per_tile, "peak_intersection_bytes": int(peak_list_bytes),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out))


COPY_BYTES = 1 << 30


def copy_probe(torch, dev, reps=5):
    """Device-to-device copy of 1 GiB (read + write counted): the achievable
    HBM rate, and the known-size dispatch that calibrates the traffic
    counters."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2 * COPY_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def traffic_summary(fetch_dir, write_dir, workload, command):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every library kernel from
    two counter runs, scaled by what the same counters read for the 1 GiB
    copy (the largest copy dispatch), written as a table under profiles/."""
    import csv
    import glob

    def load(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert files, f"no counter_collection.csv under {d}"
        per = {}
        for f in files:
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if row["Counter_Name"] != counter:
                        continue
                    per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return per

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_name = [k for k in fetch if "copyBuffer" in k or "copy" in k.lower()]
    assert copy_name, "the copy dispatch is missing from the counter run"
    cf = max(max(fetch[k]) for k in copy_name)
    cw = max(max(write.get(k, [0.0])) for k in copy_name)
    f_scale = (COPY_BYTES / 1024.0) / cf
    w_scale = (COPY_BYTES / 1024.0) / cw
    rows = []
    for name in sorted(fetch):
        short = name.split("(")[0].replace("void ", "").replace("gs::", "")
        base = short.split("<")[0]
        if not base.startswith("k_"):
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write.get(name, [0.0])) / max(1, len(write.get(name, [])))
        total = int(round((fk * f_scale + wk * w_scale) * 1024.0))
        digest = kernel_digest(base) if base in KERNEL_SOURCES else "-"
        rows.append(f"| {base} | {len(fetch[name])} | {fk:.1f} | {wk:.1f} | {total} | {digest} |")
    text = [f"# HBM traffic per dispatch, {workload}", "",
            "Two counter runs of the same benchmark command, one counter each:", "",
            "    " + command.replace("COUNTER", "FETCH_SIZE"),
            "    " + command.replace("COUNTER", "WRITE_SIZE"), "",
            f"Calibration: the 1 GiB device copy read {cf:.1f} KiB (FETCH_SIZE) and wrote {cw:.1f} KiB "
            f"(WRITE_SIZE) against {COPY_BYTES // 1024} KiB each way: scale factors {f_scale:.4f} and "
            f"{w_scale:.4f}.", "",
            "The digest column is a hash of the kernel's sources when the counters were taken; the "
            "benchmark reports the bytes only while it matches.", "",
            "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | sources digest |",
            "|---|---|---|---|---|---|"] + rows
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(workload), "w") as fh:
        fh.write("\n".join(text) + "\n")
    print(traffic_file(workload))


def cpu_baseline(cfg, params_np, cams, sample_views):
    """The oracle's full step (preprocess .. Adam) on `sample_views` of the
    workload's views with all Gaussians, on this host's cores; the rate is
    scaled to the full batch of views (the oracle's work is per view except
    the Adam update, which it runs once)."""
    import numpy as np

    from gaussian_splatting_differentiable_ewa_amd import scenes as S
    from oracle import oracle as O

    sub = cams[:sample_views]
    target = np.random.default_rng(cfg.target_seed).random((len(sub), 3, sub[0].height, sub[0].width),
                                                           dtype=np.float32)
    t0 = time.perf_counter()
    O.train_step(params_np, cfg.sh_degree, sub, target, cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, 1)
    dt = time.perf_counter() - t0
    per_step = dt * len(cams) / len(sub)
    cores = os.cpu_count()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = int(omp) if omp and omp.isdigit() else cores
    return {"value": round(1.0 / per_step, 5), "unit": "iter/s", "cores": threads, "kind": "oracle",
            "sample": f"full step on {len(sub)} of {len(cams)} views ({dt:.1f}s), all {cfg.n} Gaussians, "
                      f"scaled x{len(cams) / len(sub):g} to the batch"}


if __name__ == "__main__":
    main()
