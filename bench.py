"""Benchmark: one training step (preprocess, keys, sort, ranges, forward
raster, L1 loss, backward raster, preprocess backward, Adam) of the tile-based
differentiable Gaussian rasterizer on one MI355X.

Workload (default): 1M Gaussians, SH degree 3, a batch of 4 views at
1920x1080 (yaw 0/5/10/15 degrees about the scene centre), L1 against the render
of a second seeded scene, fp32. Inputs are synthetic and resident in HBM before
timing; `--config` picks one of the other four scenes.

Prints one JSON line. `value` is iterations/s of the whole step, Mpix/s and
the per-stage breakdown ride along.

* `step_hbm_fraction`: the method's algorithmic bytes per step (the plain
  per-stage byte model: each stage of the unfused pipeline reads its inputs
  and writes its outputs once, dense Adam over all Gaussians) with the
  measured intersection and visibility counts, over the step time, over
  8 TB/s. `step_hbm_fraction_impl` uses the bytes this implementation's fused
  passes must move (no image round trips, Adam only over the Gaussians whose
  state flags say their update is not the identity), with its terms listed.
* `roofline`: the step's dominant kernel, timed with HIP events on the stream
  it runs on. For a raster kernel the bound is the fp32 ALUs: 12 flops per
  evaluated (pixel, entry) pair per walk -- every entry of a pixel's list up
  to its last contributor, summed from n_contrib -- against the published
  157.3 TFLOP/s (packed two-wide fp32; the rate without packed instructions,
  which this build does not emit, is given beside it); for the others,
  algorithmic HBM bytes against 8 TB/s. `traffic` is the kernel's measured HBM
  bytes per dispatch from the committed counter summary (null once its sources
  have changed).
* `cpu_baseline`: the CPU oracle's whole step on the same workload, timed on
  this host, per stage; on the two small scenes also on one thread.

Subcommands turn rocprofv3 output into the summaries under profiles/
(`--stats-summary`, `--traffic-summary`, `--counters-summary`).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
# published fp32 vector rate (256 CUs x 64 lanes x 2 flops (fma) x 2 (packed
# two-wide) x 2.4 GHz); the same without packed fp32 instructions, which this
# build does not emit
FP32_PEAK_TFLOPS = 157.3
FP32_NONPACKED_TFLOPS = 78.6
# fp32 operations every evaluated (pixel, entry) pair costs in a raster walk:
# dx, dy (2), the power polynomial (3 mul + 2 fma = 7), exp (1), opacity x G
# (1), the 0.99 clamp (1)
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
    "k_preprocess": ["preprocess.hip", "project.h", "internal.h", "common.h"],
    "k_tile_masks": ["tile_masks.hip", "raster_common.h", "internal.h", "common.h"],
    "k_tl_sort": ["tile_lists.hip", "raster_common.h", "internal.h", "common.h"],
    "k_bin_fill": ["tile_lists.hip", "internal.h", "common.h"],
    "k_bin_count": ["tile_lists.hip", "internal.h", "common.h"],
}
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30


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
            parts = [p.strip() for p in line.strip().strip("|").split("|")]
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
    ap.add_argument("--lists", choices=["auto", "binned", "radix", "compact"], default="auto",
                    help="list builder: binning per tile, the global key sort, binning of the Gaussians each view "
                         "sees, or chosen per scene")
    ap.add_argument("--no-state-flags", action="store_true",
                    help="dense Adam: read every Gaussian's moments, also those known to be zero and unseen")
    ap.add_argument("--generated-order", action="store_true",
                    help="keep the Gaussians in the generated (random) order instead of the Morton order of their means")
    ap.add_argument("--separate-raster", action="store_true",
                    help="forward + loss and backward raster as two passes instead of the fused one")
    ap.add_argument("--separate-backward", choices=["visible", "compact", "dense"], default=None,
                    help="the preprocess backward and Adam as two calls instead of the fused pass: the gradient "
                         "written for the Gaussians seen in the step only (a [P][n] buffer with visibility flags, "
                         "or their columns stored consecutively), or for every Gaussian")
    ap.add_argument("--band-rows", type=int, default=None,
                    help="memory-capped mode: lists and raster one window of this many tile rows at a time")
    ap.add_argument("--list-budget", type=float, default=None, metavar="MB",
                    help="memory-capped mode: windows of tile rows planned so that the intersection lists and "
                         "their workspace stay under this many MB (1e6 bytes)")
    ap.add_argument("--moving-camera", type=float, default=0.0, metavar="DEG",
                    help="turn every camera by this many degrees about its vertical axis after each step, so "
                         "that the visible set changes from step to step (timed steps included)")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "NAME"),
                    help="no benchmark: turn a rocprofv3 --stats kernel_stats.csv into profiles/NAME.md")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no benchmark: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, csv output) into the traffic summary under profiles/")
    ap.add_argument("--counters-summary", nargs="+", metavar="DIR",
                    help="no benchmark: turn rocprofv3 --pmc runs (SQ counters, csv output) into "
                         "profiles/counters_<workload>.md")
    ap.add_argument("--runs-summary", nargs="+", metavar="JSON",
                    help="no benchmark: turn output lines of this script (one file each) into "
                         "profiles/bench_runs.md; the command of a line is its own 'argv' field, else the "
                         "--command given for that file, in order")
    ap.add_argument("--command", action="append", default=[],
                    help="for the summaries: a command that produced the profiler output (repeatable; "
                         "quoted in the summary)")
    ap.add_argument("--note", default="", help="for the summaries: a paragraph on what the run covers")
    return ap.parse_args()


# ---- byte models -------------------------------------------------------------
def method_bytes(P, n, K_v, N_v, n_any, n_px):
    """Algorithmic HBM bytes per stage of one step of the method as a pipeline
    of separate stages (each reads its inputs and writes its outputs once; a
    48-byte record and 36-byte 2D gradients per visible (view, Gaussian); dense
    Adam over all n), from the measured intersections K_v and visible
    Gaussians N_v per view, those visible in any view n_any, and pixels per
    view n_px:
      preprocess      12 n + (Bp - 12) n_any + sum_v (48 N_v + 4 n)
      scan            sum_v 8 n
      emit            sum_v (16 N_v + 12 K_v)
      sort            sum_v 24 K_v
      ranges          sum_v 8 K_v
      raster_fwd      sum_v (4 K_v + 36 N_v + 20 n_px)
      loss            sum_v 36 n_px
      raster_bwd      sum_v (4 K_v + 36 N_v + 20 n_px + 72 N_v)
      preprocess_bwd  Bp n_any + sum_v 84 N_v + Bp n
      adam            7 Bp n
    with Bp = 4 P the parameter bytes of a Gaussian."""
    Bp = 4 * P
    V = len(N_v)
    K, Nv = sum(K_v), sum(N_v)
    return {
        "preprocess": 12 * n + (Bp - 12) * n_any + 48 * Nv + 4 * V * n,
        "scan": 8 * V * n,
        "emit": 16 * Nv + 12 * K,
        "sort": 24 * K,
        "ranges": 8 * K,
        "raster_fwd": 4 * K + 36 * Nv + 20 * V * n_px,
        "loss": 36 * V * n_px,
        "raster_bwd": 4 * K + 36 * Nv + 20 * V * n_px + 72 * Nv,
        "preprocess_bwd": Bp * n_any + 84 * Nv + Bp * n,
        "adam": 7 * Bp * n,
    }


def impl_bytes(P, n, V, K, Nv, n_any, n_px, n_adam=None):
    """The bytes this implementation's stages must move (each input read once,
    each output written once), per stage of the step driver. n_adam: the
    Gaussians the fused backward + Adam must read and update (all n, unless the
    per-Gaussian state flags mark some with zero moments and no gradient,
    whose update is the identity and moves nothing)."""
    n_adam = n if n_adam is None else n_adam
    Bp = 4 * P
    return {
        # means for culling, the rest for Gaussians visible anywhere; per
        # visible pair a 48-byte record, an 8-byte rectangle, a 4-byte depth
        # copy and its 36-byte 2D-gradient record zeroed; a count per pair
        # (the global key sort's path, which then scans them: "scan"), or
        # per wave of 64 Gaussians a 4-byte sum of its counts (the binned
        # path: only the total is formed)
        "preprocess": 12 * n + (Bp - 12) * n_any + (48 + 8 + 4 + 36) * Nv + 4 * V * n,
        "preprocess_total": 12 * n + (Bp - 12) * n_any + (48 + 8 + 4 + 36) * Nv + 4 * ((n + 63) // 64),
        "scan": 8 * V * n,
        # the binned lists: rectangles and depths of visible pairs read twice
        # (count, fill), an id and a 16-bit sub-block mask written per
        # intersection, each sorted through LDS (read + write of depth and
        # id), ranges; the masks' record gathers are cache traffic
        "intersections": 2 * 12 * Nv + (8 + 8) * K + (4 + 2) * K + 8 * V * n_px // 256,
        # the "compact" builder's sets: every pair's rectangle read twice
        # (count, write), each seen Gaussian's index written
        "visible_sets": 2 * 8 * V * n + 4 * Nv,
        # the three global-sort stages and the mask pass
        "emit": 16 * V * n + 12 * K,
        "sort": 24 * K,
        "ranges": 8 * K,
        "tile_masks": (4 + 48 + 2) * K,
        # forward raster with the L1 loss: ids and masks, one record read per
        # visible pair, target read, T_final + n_contrib + dL/dimage written
        "raster_fwd_loss": 6 * K + 36 * Nv + 32 * V * n_px,
        "raster_bwd": 6 * K + 36 * Nv + 32 * V * n_px + 36 * Nv,
        # the two raster passes and the loss in one: ids and masks, one record
        # read per visible pair, target read, 2D gradients written
        "raster_fwd_bwd": 6 * K + 36 * Nv + 12 * V * n_px + 36 * Nv,
        "preprocess_bwd": Bp * n_any + 44 * Nv + Bp * n,
        "adam": 7 * Bp * n,
        # the separate pair with the gradient of the seen Gaussians only: their
        # parameters read and gradient columns written (and a visibility byte
        # per Gaussian); Adam reads those columns and the visibility (the
        # flags, or every rectangle) and updates the n_adam Gaussians; the
        # compact form's list of seen Gaussians (rectangles read twice)
        "preprocess_bwd_visible": Bp * n_any + 44 * Nv + Bp * n_any + n,
        "adam_visible": n + Bp * n_any + 6 * Bp * n_adam,
        "preprocess_bwd_compact": 2 * 8 * V * n + 4 * n_any + Bp * n_any + 44 * Nv + Bp * n_any,
        "adam_compact": 8 * V * n + 4 * n_any + Bp * n_any + 6 * Bp * n_adam,
        # the two above in one pass: every (view, Gaussian) rectangle and each
        # visible pair's 2D gradient read, the gradient never stored; for each
        # Gaussian updated, parameters and moments read once, parameters and
        # moments written
        "preprocess_bwd_adam": 8 * V * n + 36 * Nv + 6 * Bp * n_adam,
    }


# ---- the benchmark ---------------------------------------------------------------
def main():
    args = parse()
    if args.runs_summary:
        return runs_summary(args.runs_summary, args.command, args.note)
    if args.stats_summary:
        return stats_summary(args.stats_summary[0], args.stats_summary[1], args.command, args.note)
    if args.traffic_summary:
        from gaussian_splatting_differentiable_ewa_amd import scenes as S
        return traffic_summary(args.traffic_summary[0], args.traffic_summary[1], S.CONFIGS[args.config].name,
                               args.command, args.note)
    if args.counters_summary:
        from gaussian_splatting_differentiable_ewa_amd import scenes as S
        return counters_summary(args.counters_summary, S.CONFIGS[args.config].name, args.command, args.note)
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
    if perm is not None:
        params_np = np.ascontiguousarray(params_np[:, perm])
    params = torch.from_numpy(params_np).to(dev)
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    ts = TrainStep(params.clone(), cfg.sh_degree, cams, target, lr=cfg.lr, betas=(cfg.beta1, cfg.beta2),
                   eps=cfg.eps, band_rows=args.band_rows, fused_raster=not args.separate_raster, lists=args.lists,
                   state_flags=not args.no_state_flags,
                   list_budget=int(args.list_budget * 1e6) if args.list_budget else None,
                   fused_adam=args.separate_backward is None,
                   sparse_grad={"visible": True, "compact": "compact", "dense": False}.get(args.separate_backward,
                                                                                         False))
    print(f"[bench] {cfg.name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    b = ts.buf
    names = ts.stage_names
    turn = [0.0]

    def advance_cameras():
        if args.moving_camera:
            turn[0] += args.moving_camera
            b.cams = [turned(c, turn[0]) for c in cams]

    for _ in range(args.warmup):
        ts.step()
        advance_cameras()
    ts.flush()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t0_applied, redone0 = ts.t, ts.redone
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        ts.step(marks=events[k])
        if args.moving_camera:
            advance_cameras()
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
    n_px = H * W
    mpix = V * n_px * it_s / 1e6

    # the counts of the last step (its cameras)
    rect = b.rect.view(V, b.n, 4).cpu().numpy().view(np.uint16).astype(np.int64)
    vis = (rect[..., 2] > rect[..., 0]) & (rect[..., 3] > rect[..., 1])
    n_vis = [int(x) for x in vis.sum(axis=1)]
    K_v = [int(x) for x in np.where(vis, (rect[..., 2] - rect[..., 0]) * (rect[..., 3] - rect[..., 1]), 0).sum(axis=1)]
    n_any = int(vis.any(axis=0).sum())
    K = sum(K_v)
    # with the state flags on, the fused backward + Adam touches only the
    # Gaussians whose moments are not known to be zero (those seen so far)
    n_adam = int((ts.adam_state != 0).sum()) if (ts.fused_adam or ts.sparse_grad) and ts._use_state else b.n
    mb = method_bytes(b.P, b.n, K_v, n_vis, n_any, n_px)
    step_bytes = sum(mb.values())
    frac_step = step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9)
    ib = impl_bytes(b.P, b.n, V, K, sum(n_vis), n_any, n_px, n_adam)
    used = ["preprocess"] + (["scan"] if b.with_offsets else [])
    if ts.windowed or b.binned:
        used.append("intersections")
        if b.path == "compact" and not ts.windowed:
            used.append("visible_sets")
    else:
        used += ["emit", "sort", "ranges", "tile_masks"]
    used += ["raster_fwd_bwd"] if ts.fused_raster else ["raster_fwd_loss", "raster_bwd"]
    sep = {None: "", "visible": "_visible", "compact": "_compact", "dense": ""}[args.separate_backward]
    # a stage's impl term under the stage's own name (the separate backward's
    # sparse forms have their own byte counts)
    stage_term = {"preprocess_bwd": "preprocess_bwd" + sep, "adam": "adam" + sep,
                  "preprocess": "preprocess" if b.with_offsets else "preprocess_total"}
    used += ["preprocess_bwd_adam"] if ts.fused_adam else ["preprocess_bwd", "adam"]
    impl_terms = {k: int(ib[stage_term.get(k, k)]) for k in used}
    ib = {k: ib[stage_term.get(k, k)] for k in ib}
    impl_total = sum(impl_terms.values())

    # dominant kernel: the single-kernel stage with the largest time
    pairs = ts.evaluated_pairs()  # (pixel, entry) pairs up to each last contributor (after the timed steps)
    single = {"raster_fwd_loss": "k_raster_fwd_l1", "raster_bwd": "k_raster_bwd", "adam": "k_adam",
              "preprocess_bwd": "k_preprocess_bwd", "preprocess_bwd_adam": "k_preprocess_bwd",
              "raster_fwd_bwd": "k_raster_fwd_bwd_l1"}
    if args.separate_backward == "visible":
        single["adam"] = "k_adam_visible"
    elif args.separate_backward == "compact":
        del single["adam"], single["preprocess_bwd"]  # two kernels each (the seen list; listed and unlisted)
    single = {k: v for k, v in single.items() if k in stage_ms}
    dom = max(single, key=lambda k: stage_ms[k])
    kern = single[dom]
    dur_s = stage_ms[dom] * 1e-3
    if dom.startswith("raster"):
        # the fused pass evaluates every pair twice (forward, then backward)
        per_pair = FLOPS_PER_PAIR * (2 if dom == "raster_fwd_bwd" else 1)
        flops = per_pair * pairs
        achieved = flops / dur_s / 1e12
        roofline = {"bound": "alu", "kernel": kern, "achieved": round(achieved, 3), "peak": FP32_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 4),
                    "traffic": stored_traffic(cfg.name, kern),
                    "peak_nonpacked": FP32_NONPACKED_TFLOPS,
                    "frac_nonpacked": round(achieved / FP32_NONPACKED_TFLOPS, 4),
                    "algorithmic_flops": flops, "pairs": pairs, "flops_per_pair": per_pair,
                    "algorithmic_bytes": int(ib[dom]), "hbm_gbs_algorithmic": round(ib[dom] / dur_s / 1e9, 1)}
    else:
        achieved = ib[dom] / dur_s / 1e9
        roofline = {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": stored_traffic(cfg.name, kern), "algorithmic_bytes": int(ib[dom])}
    roofline["avg_launch_ms"] = round(stage_ms[dom], 4)

    # intersection statistics; in the memory-capped mode the ranges buffer
    # holds only the last window's tiles
    n_rng = b.V * b.TX * ts.windows[-1][1] if ts.windowed else b.V * b.T
    rng_ = b.ranges.view(-1, 2)[:n_rng].to(torch.int64)
    max_per_tile = int((rng_[:, 1] - rng_[:, 0]).max())
    peak_list_bytes = ts.list_bytes()
    copy_gbs = copy_probe(torch, L, dev)
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        # the oracle on the same step: the last step's cameras, the GPU's target
        bcams = list(b.cams)
        tgt = target.cpu().numpy()
        cpu = cpu_baseline(cfg, params_np, bcams, tgt)
        if args.config in (0, 1):
            cpu1 = cpu_baseline(cfg, params_np, bcams, tgt, threads=1)

    out = {
        "argv": "python bench.py " + " ".join(sys.argv[1:]),
        "metric": METRIC, "value": round(it_s, 3), "unit": "iter/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "gaussians": cfg.n, "sh_degree": cfg.sh_degree, "views": V,
                   "width": W, "height": H},
        "mpix_per_s": round(mpix, 2),
        "step_hbm_fraction": round(frac_step, 4), "step_algorithmic_bytes": int(step_bytes),
        "step_bytes_by_stage": {k: int(v) for k, v in mb.items()},
        "step_hbm_fraction_impl": round(impl_total / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "step_impl_bytes": impl_total, "step_impl_bytes_by_stage": impl_terms,
        "intersections": K, "intersections_per_view": K_v, "k_per_gaussian": round(K / b.n, 4),
        "list_builder": b.path, "band_rows": args.band_rows, "list_budget_mb": args.list_budget,
        "windows": [list(w) for w in ts.windows] if ts.windowed else None,
        "raster": "separate" if args.separate_raster else "fused",
        "backward": args.separate_backward or "fused",
        "grad_buffer_bytes": int(ts.grad.numel() * 4) if ts.grad is not None else 0,
        "gaussian_order": "generated" if args.generated_order else "morton",
        "adam_state_flags": bool(ts._use_state), "camera_turn_deg_per_step": args.moving_camera,
        "host_count_read": not ts.defer_count or not b.lists_without_count(), "redone_steps": redone,
        "visible_per_view": n_vis, "visible_any_view": n_any, "adam_gaussians": n_adam,
        "max_per_tile": max_per_tile, "peak_intersection_bytes": int(peak_list_bytes),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    if cpu1 is not None:
        out["cpu_baseline_1thread"] = cpu1
    print(json.dumps(out))


def turned(cam, deg):
    """`cam` turned by `deg` degrees about its own vertical (y) axis."""
    import numpy as np

    from gaussian_splatting_differentiable_ewa_amd import scenes as S
    th = math.radians(deg)
    c, s = math.cos(th), math.sin(th)
    R = np.asarray(cam.R, np.float64).reshape(3, 3)
    t = np.asarray(cam.t, np.float64)
    pos = -R.T @ t
    # camera to world turned by a yaw about the world y axis at the camera
    yaw = np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]])
    R2 = (yaw @ R.T).T
    t2 = -R2 @ pos
    return S.Camera(width=cam.width, height=cam.height, fx=cam.fx, fy=cam.fy, cx=cam.cx, cy=cam.cy,
                    R=tuple(float(np.float32(v)) for v in R2.reshape(-1)),
                    t=tuple(float(np.float32(v)) for v in t2), near=cam.near, far=cam.far)


def copy_probe(torch, L, dev, reps=5):
    """The library's plain device copy of 1 GiB (read + write counted): the
    achievable HBM rate, and the known-size dispatch that calibrates the
    traffic counters."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    L.gs_stream_copy(dst, src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        L.gs_stream_copy(dst, src)
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(dst[:1024], src[:1024])
    return 2 * COPY_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, params_np, cams, target, threads=None):
    """The CPU oracle's whole step (preprocess, emit + sort of the keys,
    ranges, forward, L1 loss, backward, preprocess backward, Adam) on all views
    and Gaussians of the workload, on this host, each stage timed; `threads`
    limits the oracle's OpenMP threads (all host threads by default)."""
    import numpy as np

    from oracle import oracle as O

    if threads is not None:
        O.set_threads(threads)
    try:
        used = O.max_threads()
        st = {}
        clock = time.perf_counter
        t_all = clock()

        def done(stage, t_stage):
            st[stage] = clock() - t_stage
            print(f"[bench] oracle {stage}: {st[stage]:.2f} s ({used} threads)", file=sys.stderr, flush=True)

        t = clock()
        proj = O.preprocess(params_np, cfg.sh_degree, cams)
        done("preprocess", t)
        rect, vis, z = O.rects(proj)
        t = clock()
        keys, _ = O.emit_sorted(rect, vis, z, cams[0].tiles_x, cams[0].tiles_y)
        done("emit_sort", t)
        t = clock()
        O.tile_ranges(keys, len(cams) * cams[0].n_tiles)
        done("ranges", t)
        t = clock()
        fwd = O.render_fwd(proj, cams)
        done("raster_fwd", t)
        t = clock()
        _, dL = O.loss_l1(fwd["image"], target)
        done("loss", t)
        t = clock()
        g2 = O.render_bwd(proj, cams, dL)
        done("raster_bwd", t)
        t = clock()
        grad = O.preprocess_bwd(params_np, cfg.sh_degree, cams, g2)
        done("preprocess_bwd", t)
        z0 = np.zeros_like(params_np)
        t = clock()
        O.adam(params_np, grad.astype(np.float32), z0, z0, cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, 1)
        done("adam", t)
        total = clock() - t_all
    finally:
        if threads is not None:
            O.set_threads(os.cpu_count() or 1)
    cores = os.cpu_count()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return {"value": round(1.0 / total, 5), "unit": "iter/s", "cores": used, "kind": "oracle",
            "sample": f"one whole step of the workload ({len(cams)} views, all {cfg.n} Gaussians, the GPU's "
                      f"target): {total:.1f} s on {used} OpenMP threads ({cores} host threads available)",
            "cpu_model": cpu_model(), "host_threads": cores, "stages_s": {k: round(v, 3) for k, v in st.items()}}


# ---- profile summaries -----------------------------------------------------------
def _short(name):
    s = name.split("(")[0].replace("gs::", "")
    return s[5:] if s.startswith("void ") else s


def _header(title, commands, note):
    text = [f"# {title}", "", "Produced by `bench.py` from the output of these commands (repository root, one "
            "MI355X):", ""] + ["    " + c for c in commands] + [""]
    if note:
        text += [note, ""]
    return text


def runs_summary(files, commands, note):
    """One row per benchmark line (the last line of each file): workload and
    options, it/s, ms, Mpix/s, the step's HBM fractions, the stages, the
    dominant kernel's roofline fraction, and the CPU oracle's whole step."""
    rows, cmds = [], []
    for i, path in enumerate(files):
        with open(path) as fh:
            d = json.loads(fh.read().strip().splitlines()[-1])
        cmd = d.get("argv") or (commands[i] if i < len(commands) else "?")
        cmds.append(cmd)
        opts = []
        if d.get("list_budget_mb"):
            opts.append(f"budget {d['list_budget_mb']:g} MB, {len(d['windows'])} windows")
        if d.get("band_rows"):
            opts.append(f"windows of {d['band_rows']} rows")
        if d.get("raster") == "separate":
            opts.append("separate raster")
        if d.get("gaussian_order") == "generated":
            opts.append("generated order")
        if not d.get("adam_state_flags"):
            opts.append("dense Adam")
        if d.get("camera_turn_deg_per_step"):
            opts.append(f"camera {d['camera_turn_deg_per_step']:g} deg/step")
        if d.get("backward", "fused") != "fused":
            opts.append(f"separate backward ({d['backward']} gradient, {d['grad_buffer_bytes'] / 1e6:.0f} MB)")
        opts.append(d.get("list_builder", ""))
        rf = d["roofline"]
        cpu = d.get("cpu_baseline") or {}
        cpu1 = d.get("cpu_baseline_1thread") or {}
        cpu_s = f"{1.0 / cpu['value']:.2f} s ({cpu['cores']} thr)" if cpu else "-"
        if cpu1:
            cpu_s += f"; {1.0 / cpu1['value']:.2f} s (1 thr)"
        stages = ", ".join(f"{k} {v:.3f}" for k, v in d["stages_ms"].items())
        rows.append(f"| {i + 1} | {d['config']['workload']} | {'; '.join(o for o in opts if o)} | {d['value']:.1f} | "
                    f"{d['ms_per_step']:.3f} | {d['mpix_per_s']:.0f} | {d['step_hbm_fraction']:.3f} | "
                    f"{d['step_hbm_fraction_impl']:.3f} | {d['k_per_gaussian']:.2f} | "
                    f"{d['peak_intersection_bytes'] / 1e6:.1f} | {d.get('redone_steps', 0)} | {stages} | "
                    f"{rf['kernel']} {rf['frac']:.3f} of {rf['peak']} {rf['unit']} | {cpu_s} |")
    text = _header("Benchmark lines (bench.py, one MI355X)", [f"({i + 1}) {c}" for i, c in enumerate(cmds)], note)
    text += ["Columns: it/s and ms per step over the timed steps; Mpix/s = views x W x H x it/s / 1e6; the step's "
             "HBM fraction with the method's per-stage bytes and with this implementation's; intersections per "
             "Gaussian; peak list bytes (MB); steps redone after a list overflow; event-timed stages (ms); the "
             "dominant kernel's roofline fraction; the CPU oracle's whole step (seconds, threads).", "",
             "| # | workload | options | it/s | ms | Mpix/s | HBM frac (method) | HBM frac (impl) | K/N | list MB | "
             "redone | stages ms | dominant kernel | CPU oracle step |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"] + rows
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, "bench_runs.md")
    with open(path, "w") as fh:
        fh.write("\n".join(text) + "\n")
    print(path)


def stats_summary(stats_csv, name, commands, note):
    """Per-kernel call counts and durations from rocprofv3 --stats
    (kernel_stats.csv) as profiles/NAME.md."""
    import csv
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    text = _header(f"rocprofv3 kernel statistics: {name}", commands, note)
    text += ["Durations in microseconds.", "", "| kernel | calls | avg us | min us | max us | total us | % |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        text.append(f"| {_short(r['Name']).replace('|', '/')[:140]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                    f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, name + ".md")
    with open(path, "w") as fh:
        fh.write("\n".join(text) + "\n")
    print(path)


def _counter_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert files, f"no counter_collection.csv under {d}"
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def traffic_summary(fetch_dir, write_dir, workload, commands, note):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every library kernel from
    two counter runs, scaled by what the same counters read for the library's
    1 GiB stream copy (k_stream_copy), written as a table under profiles/."""

    def load(d, counter):
        per = {}
        for row in _counter_rows(d):
            if row["Counter_Name"] == counter:
                per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return per

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "k_stream_copy" in k]
    assert copy, "the copy dispatch is missing from the counter run"
    cf = max(max(fetch[k]) for k in copy)
    cw = max(max(write.get(k, [0.0])) for k in copy)
    f_scale, w_scale = (COPY_BYTES / 1024.0) / cf, (COPY_BYTES / 1024.0) / cw
    rows = []
    for name in sorted(fetch):
        base = _short(name).split("<")[0]
        if not base.startswith("k_") or base == "k_stream_copy":
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write.get(name, [0.0])) / max(1, len(write.get(name, [])))
        total = int(round((fk * f_scale + wk * w_scale) * 1024.0))
        digest = kernel_digest(base) if base in KERNEL_SOURCES else "-"
        rows.append(f"| {base} | {len(fetch[name])} | {fk:.1f} | {wk:.1f} | {total} | {digest} |")
    text = _header(f"HBM traffic per dispatch, {workload}", commands, note)
    text += [f"Calibration: the library's 1 GiB stream copy (k_stream_copy) read {cf:.1f} KiB (FETCH_SIZE) and wrote "
             f"{cw:.1f} KiB (WRITE_SIZE) against {COPY_BYTES // 1024} KiB each way: scale factors {f_scale:.4f} and "
             f"{w_scale:.4f}.", "",
             "The digest column is a hash of the kernel's sources when the counters were taken; the "
             "benchmark reports the bytes only while it matches.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | sources digest |",
             "|---|---|---|---|---|---|"] + rows
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(workload), "w") as fh:
        fh.write("\n".join(text) + "\n")
    print(traffic_file(workload))


def counters_summary(dirs, workload, commands, note):
    """SQ counters per dispatch of the library's kernels (means over
    dispatches) from rocprofv3 --pmc runs, with VALU busy (instructions x 4
    cycles over 1024 SIMDs x duration x 2.4 GHz), LDS bank-conflict share,
    and the shares of wave time spent waiting and issuing."""
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for d in dirs:
        for row in _counter_rows(d):
            k = _short(row["Kernel_Name"])
            if not k.startswith("k_"):
                continue
            per[k][row["Counter_Name"]].append(float(row["Counter_Value"]))
            dur[k][(d, row.get("Dispatch_Id", row.get("Correlation_Id", "")))] = \
                (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
    text = _header(f"SQ counters per dispatch, {workload}", commands, note)
    text += ["Per-dispatch means. VALU busy = SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x duration x 2.4 GHz); LDS "
             "conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; waiting and issuing = SQ_WAIT_ANY and "
             "SQ_ACTIVE_INST_ANY over SQ_WAVE_CYCLES. Durations are those of the counter runs (the profiler "
             "lengthens short dispatches).", "",
             "| kernel | us | VALU instr (M) | VALU busy | LDS instr (M) | LDS conflict share | SALU instr (M) | "
             "VMEM rd (M) | waves waiting | waves issuing |", "|---|---|---|---|---|---|---|---|---|---|"]
    mean = lambda xs: sum(xs) / len(xs)
    for k in sorted(per, key=lambda k: -mean(list(dur[k].values()))):
        c = {n: mean(v) for n, v in per[k].items()}
        d = mean(list(dur[k].values()))
        g = lambda n, sc=1.0: f"{c[n] / sc:.1f}" if n in c else "-"
        busy = f"{c['SQ_INSTS_VALU'] * 4 / (1024 * d * 2.4e9):.2f}" if "SQ_INSTS_VALU" in c else "-"
        conf = (f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.3f}"
                if c.get("SQ_LDS_IDX_ACTIVE") else "-")
        share = lambda n: f"{c[n] / c['SQ_WAVE_CYCLES']:.2f}" if n in c and c.get("SQ_WAVE_CYCLES") else "-"
        text.append(f"| {k} | {d * 1e6:.0f} | {g('SQ_INSTS_VALU', 1e6)} | {busy} | {g('SQ_INSTS_LDS', 1e6)} | {conf} | "
                    f"{g('SQ_INSTS_SALU', 1e6)} | {g('SQ_INSTS_VMEM_RD', 1e6)} | {share('SQ_WAIT_ANY')} | "
                    f"{share('SQ_ACTIVE_INST_ANY')} |")
    text += ["", "Raw means:", "", "| kernel | counter | value |", "|---|---|---|"]
    for k in sorted(per):
        for n in sorted(per[k]):
            text.append(f"| {k} | {n} | {mean(per[k][n]):.0f} |")
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"counters_{workload}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(text) + "\n")
    print(path)


if __name__ == "__main__":
    main()
