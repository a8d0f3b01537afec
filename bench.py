"""Benchmark: one step = the whole rasterizer path on one synthetic frame.

Workload: the garden-shaped scene, 1,535,033 Gaussians, SH degree 3,
1297x840 image (82 x 53 = 4346 tiles), seeded synthetic data already resident
in HBM. One step runs gs_project, gs_bin_tiles, gs_sort_keys, gs_render_fwd and
gs_render_bwd on one HIP stream. The headline value is tile-Gaussian pairs per
second over the whole step; ms per stage and a roofline fraction for the
dominant call come with it, and the CPU oracle is timed on the host beside it
(a baseline only).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd raster ms/frame and tile-pairs/sec at 1.5M Gaussians 1297×840; % roofline"

# Algorithmic work per (pixel, splat) hit, op-counted from the method's
# definition (FMA = 2 flops): forward 21 flops + 1 exp; backward 54 flops
# (including the 9 pixel-to-splat accumulations) + exp + reciprocal.
FWD_FLOPS_PER_HIT = 21
BWD_FLOPS_PER_HIT = 54
PEAK_FP32_TFLOPS = 157.3     # MI355X published fp32 vector peak
PEAK_HBM_GBS = 8000.0        # MI355X published HBM3E bandwidth


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--chunk-mode", type=int, default=1)
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the rasterizer "
              "path here is single-GPU by design.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gaussian_splatting_differentiable_amd as gsr
    import scenegen

    torch.cuda.init()
    dev = torch.device("cuda:0")
    t0 = time.time()
    sc = scenegen.make_config(args.config)
    print(f"[bench] scene {sc.name}: {sc.n} Gaussians, {sc.camera.width}x{sc.camera.height}, "
          f"generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    cam = sc.camera
    n = sc.n

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    means, ls, qs, op, sh = up(sc.means), up(sc.log_scales), up(sc.quats), up(sc.opacities), up(sc.sh)
    dL = up(sc.dL_drgb)
    r = gsr.Rasterizer(cam, device=dev, capacity=1 << 22,
                       sched=gsr.make_sched(chunk_mode=args.chunk_mode))
    r.project(means, ls, qs, op, sh, sc.sh_degree)
    npairs = r.bin_and_sort(n)
    # grow the pair buffers once with headroom so the timed loop never overflows
    r._ensure(n, max(r.capacity, npairs + npairs // 8))
    r.project(means, ls, qs, op, sh, sc.sh_degree)
    npairs = r.bin_and_sort(n)
    r.render_fwd(n, stats=True)
    torch.cuda.synchronize()
    stats = r.stats.cpu().numpy()
    hits = int(stats[0])
    plan = r.fwd_state[:8].cpu().numpy().view(np.int32)  # (chunked tiles h, chunks k)
    chunked, chunks = int(plan[0]), int(plan[1])
    print(f"[bench] pairs {npairs}, hits {hits}, lane evaluations {int(stats[1])}, "
          f"chunked tiles {chunked} x {chunks}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    cap = r.capacity
    stages = ["project", "bin", "sort", "fwd", "bwd"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        gsr.gs_project(n, means, ls, qs, op, sh, sc.sh_degree, r.cam, r.splats)
        if ev is not None:
            ev[1].record(stream)
        gsr.gs_bin_tiles(n, r.splats, r.cam, cap, r.offsets, None, None, r.status, r.workspace)
        if ev is not None:
            ev[2].record(stream)
        gsr.gs_sort_keys(n, r.splats, r.offsets, cap, r.cam, None, r.sorted_ids, r.ranges,
                         r.workspace)
        if ev is not None:
            ev[3].record(stream)
        gsr.gs_render_fwd(n, r.splats, r.sorted_ids, r.ranges, r.cam, r.sched, r.rgb, r.T, r.last,
                          r.fwd_state, None, r.workspace)
        if ev is not None:
            ev[4].record(stream)
        gsr.gs_render_bwd(n, r.splats, r.sorted_ids, r.ranges, r.cam, r.T, r.last, r.fwd_state,
                          dL, r.grads, r.workspace)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    status = int(r.status.item())
    if status != gsr.GS_OK:
        raise SystemExit(f"pair buffer overflow during the timed loop: {gsr.strerror(status)}")

    per = {s: [] for s in stages}
    for ev in events:
        for i, s in enumerate(stages):
            per[s].append(ev[i].elapsed_time(ev[i + 1]))
    ms = {s: float(np.mean(v)) for s, v in per.items()}
    ms_min = {s: float(np.min(v)) for s, v in per.items()}
    ms_step = t_wall * 1e3 / args.steps
    ms_raster = ms["fwd"] + ms["bwd"]

    # roofline of the dominant call
    dom = max(("fwd", "bwd"), key=lambda s: ms[s])
    flops = (BWD_FLOPS_PER_HIT if dom == "bwd" else FWD_FLOPS_PER_HIT) * hits
    achieved = flops / (ms[dom] * 1e-3) / 1e12
    roofline = {"bound": "alu", "kernel": f"gs_render_{dom}", "achieved": round(achieved, 3),
                "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "traffic": None}
    raster_flops = (FWD_FLOPS_PER_HIT + BWD_FLOPS_PER_HIT) * hits
    raster_frac = raster_flops / (ms_raster * 1e-3) / 1e12 / PEAK_FP32_TFLOPS

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tc = time.perf_counter()
        o = oracle.frame(sc)
        t_cpu = time.perf_counter() - tc
        cpu = {"value": round(len(o["sorted_ids"]) / t_cpu, 1), "unit": "tile-pairs/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"one whole frame of the same scene (project, bin, sort, forward, "
                         f"backward; {t_cpu:.2f} s)"}

    line = {
        "metric": METRIC,
        "value": round(npairs / (ms_step * 1e-3), 1),
        "unit": "tile-pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{sc.name}: {n} Gaussians, SH degree {sc.sh_degree}, "
                               f"{cam.width}x{cam.height} image, {cam.num_tiles} tiles",
                   "pairs": npairs, "hits": hits, "chunk_mode": args.chunk_mode,
                   "chunked_tiles": chunked, "chunks_per_tile": chunks},
        "ms": {k: round(v, 4) for k, v in ms.items()},
        "ms_min": {k: round(v, 4) for k, v in ms_min.items()},
        "ms_raster_fwd_bwd": round(ms_raster, 4),
        "raster_pairs_per_s": round(npairs / (ms_raster * 1e-3), 1),
        "raster_frac_fp32_peak": round(raster_frac, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
