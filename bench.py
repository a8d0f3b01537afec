"""Benchmark: one step = the rasterizer hot path on one synthetic frame.

Workload: the garden-shaped scene, 1,535,033 Gaussians, SH degree 3,
1297x840 image (82 x 53 = 4346 tiles), seeded synthetic data already resident
in HBM. A step runs gs_bin_tiles, gs_sort_keys_plan (the sort, with the tile
schedule built in a spare workgroup of its last pass; frames whose last pass
is too short to hide it build it beside the sort on a second stream with
gs_plan_tiles), gs_render_fwd_zero (the forward, which checks that schedule in
its own launch and clears the gradient rows in its workers' idle end) and
gs_render_bwd_accumulate, over the projected splats. gs_project (the feeder) is
timed in its own loop and reported beside it. The
headline value is tile-Gaussian pairs per second over the step. The roofline
object covers the longest raster kernel, with algorithmic work per unit as
defined below, and the CPU oracle is timed on the host beside it (a baseline
only).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd raster ms/frame and tile-pairs/sec at 1.5M Gaussians 1297×840; % roofline"

# Algorithmic work per unit, op-counted from the method's definition (FMA = 2
# flops). Per (pixel, splat) hit: forward 21 flops + 1 exp; backward 54 flops
# (including the 9 pixel-to-splat accumulations) + exp + reciprocal.
FWD_FLOPS_PER_HIT = 21
BWD_FLOPS_PER_HIT = 54
# Bytes: every (tile, splat) pair reads its 48-byte record and 4-byte id; the
# forward writes 20 bytes per pixel (rgb, T, last); the backward reads them
# (dL/drgb, T, last) and adds 36 bytes of gradient per (8x8 sub-tile, splat)
# pair with at least one hit.
PAIR_BYTES = 52
PIXEL_BYTES = 20
ATOMIC_BYTES = 36
# Binning and sort move 48 B per Gaussian read + 4 B per Gaussian of offsets
# (bin), then 12 B per pair written, 12 B read and 4 B of ids written + 8 B per
# tile of ranges (sort). Projection reads 44 B per Gaussian (mean, log-scales,
# quaternion, opacity), 192 B of SH per visible Gaussian at degree 3, and writes
# its 48-byte record.
BIN_BYTES_PER_GAUSSIAN = 52
SORT_BYTES_PER_PAIR = 28
SORT_BYTES_PER_TILE = 8
PROJ_BYTES_PER_GAUSSIAN = 44 + 48
# The projection's backward reads the 36 B of screen-space gradients of every
# Gaussian, the 44 B of parameters of every Gaussian whose gradient row is not
# all zero (a Gaussian no pixel touched has zero gradients throughout) and its
# SH (12 B per coefficient) when it is also visible, and writes 44 B of
# parameter gradients and the SH gradient of every Gaussian (zeros for culled
# and untouched ones).
PROJ_BWD_BYTES_PER_GAUSSIAN = 36 + 44
PROJ_BWD_BYTES_PER_TOUCHED = 44
# With the SH coefficients stored as bf16 both read 6 B per coefficient instead
# of 12; the SH gradient stays fp32.
PEAK_FP32_TFLOPS = 157.3     # MI355X published fp32 vector peak
PEAK_HBM_GBS = 8000.0        # MI355X published HBM3E bandwidth
# exp and reciprocal issue at a quarter of the fp32 lane rate:
# 256 CUs x 64 lanes / 4 x 2.4 GHz
PEAK_TRANS_GPS = 256 * 64 / 4 * 2.4

CSRC = os.path.join(ROOT, "gaussian_splatting_differentiable_amd", "csrc")
KERNEL_SOURCES = {
    "k_render_fwd": ["render_fwd.hip", "render_common.h", "gs_common.h"],
    "k_render_bwd": ["render_bwd.hip", "render_common.h", "gs_common.h", "wave_reduce.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None if there
    is none for this kernel and workload or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(kernel):
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--chunk-mode", type=int, default=1)
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-configuration diagnostics of configs 1-5")
    p.add_argument("--config-steps", type=int, default=10)
    p.add_argument("--views", type=int, default=0,
                   help="also time a batch of this many views against as many single-view "
                        "steps (below 2, the default: skip)")
    return p.parse_args()


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_frames(oracle, sc, splats, budget_s, max_frames):
    """Whole frames (bin, sort, forward, backward) through the oracle until the
    time budget is spent; returns (frames, pairs, seconds)."""
    cam = sc.camera
    W, H = cam.width, cam.height
    frames, pairs, t_total = 0, 0, 0.0
    while frames == 0 or (t_total < budget_s and frames < max_frames):
        t0 = time.perf_counter()
        offsets, keys, ids = oracle.bin_tiles(splats, W, H)
        skeys, sids = oracle.sort_pairs(keys, ids)
        ranges = oracle.tile_ranges(skeys, cam.num_tiles)
        f = oracle.render_fwd(splats, sids, ranges, W, H)
        oracle.render_bwd(splats, sids, ranges, W, H, f["last"], sc.dL_drgb)
        t_total += time.perf_counter() - t0
        frames += 1
        pairs += len(sids)
    return frames, pairs, t_total


def cpu_baseline(sc, npairs_gpu):
    """The oracle's bin, sort, forward and backward on the same scene: about
    10 s of frames on every host thread, then one frame on one thread
    (projection once, outside the clock)."""
    import oracle
    splats = oracle.project_scene(sc)
    threads = oracle.num_threads()
    frames, pairs, t_total = _oracle_frames(oracle, sc, splats, 10.0, 20)
    oracle.set_num_threads(1)
    try:
        f1, p1, t1 = _oracle_frames(oracle, sc, splats, 0.0, 1)
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(pairs / t_total, 1), "unit": "tile-pairs/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{frames} whole frames of the same scene through the oracle's bin, sort, "
                      f"forward and backward on {threads} threads ({t_total:.1f} s; "
                      f"{pairs // frames} pairs per frame, GPU {npairs_gpu}); one more frame "
                      f"on 1 thread",
            "value_1_thread": round(p1 / t1, 1), "seconds_1_thread": round(t1, 2),
            "cpu_model": cpu_model(), "cpu_count": os.cpu_count()}


def oracle_frame_counts(sc):
    """Knife-edge pixels and the exact hit and live-entry counts of one frame,
    from the oracle's fp32 decision mirror (the oracle's forward on its own
    projection, binning and sort)."""
    import oracle
    cam = sc.camera
    splats = oracle.project_scene(sc)
    offsets, keys, ids = oracle.bin_tiles(splats, cam.width, cam.height)
    skeys, sids = oracle.sort_pairs(keys, ids)
    ranges = oracle.tile_ranges(skeys, cam.num_tiles)
    f = oracle.render_fwd(splats, sids, ranges, cam.width, cam.height)
    return {"knife_pixels": int(f["knife"].sum()), "pairs": int(len(sids)),
            "hits": int(f["hits"]), "live_entries": int(f["last"].astype(np.int64).sum())}


def frame_diagnostics(gsr, sc, r, n, cus):
    """Per-frame quantities of the scene already binned, sorted and rendered by r
    (with stats): visible splats, pairs, hits, live entries (sum over pixels of
    the list entries walked before the pixel stopped), the per-tile pair counts
    and the chunk plan."""
    import torch
    ranges = r.ranges.cpu().numpy().astype(np.int64)
    Nt = ranges[:, 1] - ranges[:, 0]
    I = int(Nt.sum())
    st = r.stats.cpu().numpy()
    plan = r.fwd_state[:8].cpu().numpy().view(np.int32)
    nonempty = Nt[Nt > 0]
    return {
        "gaussians": n, "visible": int((r.splats[:n, 9] > 0).sum().item()), "pairs": I,
        "hits": int(st[0]), "live_entries": int(r.last.to(torch.int64).sum().item()),
        "lane_evaluations": int(st[1]), "subtile_hits": int(st[2]),
        "tiles": int(len(Nt)), "tiles_empty": int((Nt == 0).sum()),
        "pairs_per_tile": {"max": int(Nt.max(initial=0)), "min": int(Nt.min(initial=0)),
                           "mean": round(float(Nt.mean()) if len(Nt) else 0.0, 2),
                           "min_nonempty": int(nonempty.min()) if len(nonempty) else 0},
        # the load-imbalance page's ratio of the heaviest tile to the mean work of
        # one compute unit (K = the device's compute units)
        "imbalance_nmax_over_I_per_K": round(float(Nt.max(initial=0)) / max(I / cus, 1e-9), 3),
        "chunk_plan": {"chunked_tiles": int(plan[0]), "chunks_per_tile": int(plan[1])},
    }


def make_step(gsr, r, n, dL, npairs):
    """One frame's calls on the current stream, as `step(ev=None)`: bin, sort,
    forward and backward, with HIP events ev[0..4] around them when given. The
    tile schedule is built inside the sort when the frame's last tile pass runs
    long enough to hide it (gsr.plan_in_sort), else beside the sort on a second
    stream that the forward's stream waits for; either way the forward checks
    it in its own launch. The forward clears the gradient rows in its workers'
    idle end and the backward adds into them."""
    import torch
    stream = torch.cuda.current_stream()
    planned = gsr.planned_sched(r.sched)
    in_sort = gsr.plan_in_sort(r.tiles, npairs)
    side = torch.cuda.Stream()
    ev_bin, ev_plan = torch.cuda.Event(), torch.cuda.Event()
    cap = r.capacity

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if in_sort:
            gsr.gs_bin_tiles(n, r.splats, r.cam, cap, r.offsets, None, None, r.status,
                             r.workspace)
        else:
            gsr.gs_bin_tiles(n, r.splats, r.cam, cap, r.offsets, None, None, r.status,
                             r.workspace, tile_counts=r.tile_counts)
            ev_bin.record(stream)
            side.wait_event(ev_bin)
            gsr.gs_plan_tiles(r.tile_counts, r.cam, r.sched, r.fwd_state, r.status, stream=side)
            ev_plan.record(side)
        if ev is not None:
            ev[1].record(stream)
        if in_sort:
            gsr.gs_sort_keys_plan(n, r.splats, r.offsets, cap, r.cam, None, r.sorted_ids,
                                  r.ranges, r.sched, r.fwd_state, r.status, r.workspace)
        else:
            gsr.gs_sort_keys(n, r.splats, r.offsets, cap, r.cam, None, r.sorted_ids, r.ranges,
                             r.status, r.workspace)
        if ev is not None:
            ev[2].record(stream)
        if not in_sort:
            stream.wait_event(ev_plan)
        gsr.gs_render_fwd_zero(n, r.splats, r.sorted_ids, r.ranges, r.cam, planned, r.rgb, r.T,
                               r.last, r.fwd_state, None, None, r.status, r.grads[:n])
        if ev is not None:
            ev[3].record(stream)
        gsr.gs_render_bwd_accumulate(n, r.splats, r.sorted_ids, r.ranges, r.cam, 1, r.T, r.last,
                                     r.fwd_state, dL, r.grads, r.status)
        if ev is not None:
            ev[4].record(stream)

    return step, in_sort


def stage_times(gsr, r, n, dL, steps, warmup):
    """Median ms of bin, sort (with the tile schedule built inside it or beside
    it), forward and backward over `steps` frames, HIP events between the calls."""
    import torch
    npairs = int(r.offsets[n:n + 1].item())
    step, _ = make_step(gsr, r, n, dL, npairs)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    st = int(r.status.item())
    if st != gsr.GS_OK:
        raise SystemExit(f"a frame failed: {gsr.strerror(st)}")
    names = ["bin", "sort", "fwd", "bwd"]
    ms = {s: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs]))
          for i, s in enumerate(names)}
    return ms_step, ms


def raster_roofline(hits, npairs, pixels, sub_hits, ms_fwd, ms_bwd):
    """t_roof of render_fwd + render_bwd (the larger of the fp32 and the HBM time
    of each) over their measured time."""
    t_fwd = max(FWD_FLOPS_PER_HIT * hits / (PEAK_FP32_TFLOPS * 1e12),
                (PAIR_BYTES * npairs + PIXEL_BYTES * pixels) / (PEAK_HBM_GBS * 1e9))
    t_bwd = max(BWD_FLOPS_PER_HIT * hits / (PEAK_FP32_TFLOPS * 1e12),
                (PAIR_BYTES * npairs + PIXEL_BYTES * pixels + ATOMIC_BYTES * sub_hits)
                / (PEAK_HBM_GBS * 1e9))
    return (t_fwd + t_bwd) / ((ms_fwd + ms_bwd) * 1e-3)


def config_line(gsr, dev, cfg, args, cus):
    """One configuration: its scene, one counted frame (diagnostics), then timed
    frames (stage medians, tile-pairs per second, raster roofline fraction)."""
    import torch
    import scenegen
    sc = scenegen.make_config(cfg)
    n = sc.n
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    r = gsr.Rasterizer(sc.camera, device=dev, capacity=1 << 20)
    r.project(up(sc.means), up(sc.log_scales), up(sc.quats), up(sc.opacities), up(sc.sh),
              sc.sh_degree)
    I = r.bin_and_sort(n)
    r._ensure(n, max(r.capacity, I + I // 8))
    r.bin_and_sort(n)
    r.render_fwd(n, stats=True)
    diag = frame_diagnostics(gsr, sc, r, n, cus)
    dL = up(sc.dL_drgb)
    ms_step, ms = stage_times(gsr, r, n, dL, args.config_steps, 3)
    P = sc.camera.width * sc.camera.height
    diag.update(
        workload=f"{sc.name}: {n} Gaussians, SH degree {sc.sh_degree}, "
                 f"{sc.camera.width}x{sc.camera.height} image",
        ms_per_step=round(ms_step, 4), ms={k: round(v, 4) for k, v in ms.items()},
        tile_pairs_per_s=round(I / (ms_step * 1e-3), 1),
        raster_roofline_frac=round(raster_roofline(diag["hits"], I, P, diag["subtile_hits"],
                                                   ms["fwd"], ms["bwd"]), 4))
    del r
    torch.cuda.empty_cache()
    return sc, diag


def views_stage(args, sc, gsr, dev, means, ls, qs, op, sh):
    """The same scene seen by V cameras (the scene's own and V - 1 moved ones):
    one batch (the *_views calls: one bin, sort, forward and backward launch
    sequence for all views) against V single-view frames one after another.
    Both are timed over the same steps with the wall clock (bin, sort, forward,
    backward; the projections stay outside, as in the main step)."""
    import numpy as np
    import torch
    import scenegen
    V = args.views
    rng = np.random.default_rng(77)
    c0 = sc.camera
    M0 = np.asarray(c0.world_to_cam, np.float64).reshape(3, 4)
    cams = [c0]
    for _ in range(V - 1):
        a = rng.normal(0, 0.05, 3)
        K = np.array([[0, -a[2], a[1]], [a[2], 0, -a[0]], [-a[1], a[0], 0]])
        R = np.linalg.qr(np.eye(3) + K)[0]
        R *= np.sign(np.diag(R))[None, :]   # the rotation near the identity
        cams.append(scenegen.pinhole(c0.width, c0.height, float(c0.fx),
                                     np.concatenate([R @ M0[:, :3],
                                                     (M0[:, 3] + rng.normal(0, 0.05, 3))[:, None]],
                                                    1)))
    n = sc.n
    gen = torch.Generator(device=dev).manual_seed(78)
    dL = torch.randn((3, V * c0.height, c0.width), generator=gen, device=dev)

    def grow(r, nrec):
        I = r.bin_and_sort(nrec)
        r._ensure(nrec, max(r.capacity, I + I // 8))
        return r.bin_and_sort(nrec)

    def step(r, nrec, dLv):
        # the raw calls, as in the main step (no host synchronisation inside)
        if r.V > 1:
            gsr.gs_bin_tiles_views(nrec, r.splats, r.cam, r.V, r.capacity, r.offsets, None, None,
                                   r.status, r.workspace)
            gsr.gs_sort_keys_views(nrec, r.splats, r.offsets, r.capacity, r.cam, r.V, None,
                                   r.sorted_ids, r.ranges, r.status, r.workspace)
            gsr.gs_render_fwd_views(nrec, r.splats, r.sorted_ids, r.ranges, r.cam, r.V, r.sched,
                                    r.rgb, r.T, r.last, r.fwd_state, None, None, r.status)
            gsr.gs_render_bwd_views(nrec, r.splats, r.sorted_ids, r.ranges, r.cam, r.V, r.T,
                                    r.last, r.fwd_state, dLv, r.grads, r.status)
        else:
            gsr.gs_bin_tiles(nrec, r.splats, r.cam, r.capacity, r.offsets, None, None, r.status,
                             r.workspace)
            gsr.gs_sort_keys(nrec, r.splats, r.offsets, r.capacity, r.cam, None, r.sorted_ids,
                             r.ranges, r.status, r.workspace)
            gsr.gs_render_fwd(nrec, r.splats, r.sorted_ids, r.ranges, r.cam, r.sched, r.rgb, r.T,
                              r.last, r.fwd_state, None, None, r.status)
            gsr.gs_render_bwd(nrec, r.splats, r.sorted_ids, r.ranges, r.cam, r.T, r.last,
                              r.fwd_state, dLv, r.grads, r.status)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / args.steps

    rb = gsr.Rasterizer(c0, device=dev, capacity=1 << 24, n_views=V)
    rb.project_views(cams, means, ls, qs, op, sh, sc.sh_degree)
    pairs_b = grow(rb, V * n)
    ms_b = timed(lambda: step(rb, V * n, dL))
    if int(rb.status.item()) != gsr.GS_OK:
        raise SystemExit(f"batched-views frame failed: {gsr.strerror(int(rb.status.item()))}")
    del rb
    ms_seq, pairs_seq = 0.0, 0
    H = c0.height
    for v, cam in enumerate(cams):
        r = gsr.Rasterizer(cam, device=dev, capacity=1 << 23)
        r.project(means, ls, qs, op, sh, sc.sh_degree)
        pairs_seq += grow(r, n)
        dLv = dL[:, v * H:(v + 1) * H].contiguous()
        ms_seq += timed(lambda: step(r, n, dLv))
        if int(r.status.item()) != gsr.GS_OK:
            raise SystemExit(f"single-view frame failed: {gsr.strerror(int(r.status.item()))}")
        del r
    torch.cuda.synchronize()
    return {"n_views": V, "pairs": pairs_b, "pairs_single_views": pairs_seq,
            "ms_batch_step": round(ms_b, 4), "ms_single_view_steps": round(ms_seq, 4),
            "pairs_per_s_batch": round(pairs_b / (ms_b * 1e-3), 1),
            "pairs_per_s_single_views": round(pairs_seq / (ms_seq * 1e-3), 1)}


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
    hits, lane_evals, sub_hits = int(stats[0]), int(stats[1]), int(stats[2])
    plan = r.fwd_state[:8].cpu().numpy().view(np.int32)  # (chunked tiles h, chunks k)
    chunked, chunks = int(plan[0]), int(plan[1])
    print(f"[bench] pairs {npairs}, hits {hits}, lane evaluations {lane_evals}, sub-tile hits "
          f"{sub_hits}, chunked tiles {chunked} x {chunks}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    stages = ["bin", "sort", "fwd", "bwd"]
    step, plan_in_sort = make_step(gsr, r, n, dL, npairs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    # the stage breakdown: the same steps again with HIP events between the calls
    # (kept out of the timed loop above, whose steps they would lengthen)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    # the raster kernels' own durations: the same steps again, with a pair of HIP
    # events recorded on the stream around each raster kernel launch (kept out
    # of the timed loop above, whose calls they would otherwise lengthen)
    gsr.gs_timing_start()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    kernel_ms = {"fwd": float(np.median(gsr.gs_timing_read(0))),
                 "bwd": float(np.median(gsr.gs_timing_read(1)))}
    status = int(r.status.item())  # the frames' status word, read once after all of them
    if status != gsr.GS_OK:
        raise SystemExit(f"a frame of the timed loop failed: {gsr.strerror(status)}")

    per = {s: [] for s in stages}
    for ev in events:
        for i, s in enumerate(stages):
            per[s].append(ev[i].elapsed_time(ev[i + 1]))
    ms = {s: float(np.median(v)) for s, v in per.items()}
    ms_min = {s: float(np.min(v)) for s, v in per.items()}
    ms_step = t_wall * 1e3 / args.steps

    def launch_times(call):
        """Per-launch milliseconds of `call` over args.steps launches (HIP events
        on the stream it runs on), after one untimed launch."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
        call()
        for k in range(args.steps):
            ev[2 * k].record(stream)
            call()
            ev[2 * k + 1].record(stream)
        torch.cuda.synchronize()
        return [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)]

    # the feeder and the projection's backward (the next stage of a training
    # step), each in its own loop; then both with the SH coefficients stored as
    # bf16 (the same values rounded to nearest even), the splats restored after
    K = (sc.sh_degree + 1) ** 2
    pgrads = [torch.empty(shape, dtype=torch.float32, device=dev)
              for shape in ((n, 3), (n, 3), (n, 4), (n,), (n, K, 3))]
    sh16 = sh.to(torch.bfloat16)
    per["project"] = launch_times(
        lambda: gsr.gs_project(n, means, ls, qs, op, sh, sc.sh_degree, r.cam, r.splats))
    per["project_bwd"] = launch_times(
        lambda: gsr.gs_project_bwd(n, means, ls, qs, op, sh, sc.sh_degree, r.cam, r.grads,
                                   *pgrads))
    per["project_bf16sh"] = launch_times(
        lambda: gsr.gs_project_bf16sh(n, means, ls, qs, op, sh16, sc.sh_degree, r.cam, r.splats))
    per["project_bwd_bf16sh"] = launch_times(
        lambda: gsr.gs_project_bwd_bf16sh(n, means, ls, qs, op, sh16, sc.sh_degree, r.cam,
                                          r.grads, *pgrads))
    gsr.gs_project(n, means, ls, qs, op, sh, sc.sh_degree, r.cam, r.splats)
    ms_project = float(np.median(per["project"]))
    ms_project_bwd = float(np.median(per["project_bwd"]))
    n_vis = int((r.splats[:, 9] > 0).sum().item())
    touched = (r.grads[:n] != 0).any(dim=1)
    n_touched = int(touched.sum().item())
    n_touched_vis = int((touched & (r.splats[:n, 9] > 0)).sum().item())

    # roofline of the longest raster kernel: algorithmic bytes and flops per launch
    P = cam.width * cam.height
    work = {
        "fwd": dict(flops=FWD_FLOPS_PER_HIT * hits, bytes=PAIR_BYTES * npairs + PIXEL_BYTES * P),
        "bwd": dict(flops=BWD_FLOPS_PER_HIT * hits,
                    bytes=PAIR_BYTES * npairs + PIXEL_BYTES * P + ATOMIC_BYTES * sub_hits),
    }
    t_roof = {s: max(w["flops"] / (PEAK_FP32_TFLOPS * 1e12), w["bytes"] / (PEAK_HBM_GBS * 1e9))
              for s, w in work.items()}
    dom = max(("fwd", "bwd"), key=lambda s: kernel_ms[s])
    kname = f"k_render_{dom}"
    w = work[dom]
    hbm_binds = w["bytes"] / (PEAK_HBM_GBS * 1e9) >= w["flops"] / (PEAK_FP32_TFLOPS * 1e12)
    t_s = kernel_ms[dom] * 1e-3  # the kernel's own launches, from HIP events on its stream
    traffic = measured_traffic(kname, sc.name)
    if hbm_binds:
        achieved = w["bytes"] / t_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        achieved = w["flops"] / t_s / 1e12
        roofline = {"bound": "alu", "achieved": round(achieved, 3),
                    "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "traffic": traffic}
    roofline.update(kernel=kname, kernel_ms=round(kernel_ms[dom], 4),
                    algorithmic_bytes=w["bytes"], algorithmic_flops=w["flops"],
                    fp32_frac=round(w["flops"] / t_s / 1e12 / PEAK_FP32_TFLOPS, 4))
    ms_raster = ms["fwd"] + ms["bwd"]
    raster_frac = (t_roof["fwd"] + t_roof["bwd"]) / (ms_raster * 1e-3)

    # every stage against the three ceilings: t_roof = max(F/P_F, X/P_X, B/P_B)
    sh_bytes = 4 * 3 * (sc.sh_degree + 1) ** 2
    stage_work = {
        "project": dict(flops=0, trans=0,
                        bytes=PROJ_BYTES_PER_GAUSSIAN * n + sh_bytes * n_vis),
        "project_bwd": dict(flops=0, trans=0,
                            bytes=(PROJ_BWD_BYTES_PER_GAUSSIAN + sh_bytes) * n
                            + PROJ_BWD_BYTES_PER_TOUCHED * n_touched + sh_bytes * n_touched_vis),
        "project_bf16sh": dict(flops=0, trans=0,
                               bytes=PROJ_BYTES_PER_GAUSSIAN * n + sh_bytes // 2 * n_vis),
        "project_bwd_bf16sh": dict(flops=0, trans=0,
                                   bytes=(PROJ_BWD_BYTES_PER_GAUSSIAN + sh_bytes) * n
                                   + PROJ_BWD_BYTES_PER_TOUCHED * n_touched
                                   + sh_bytes // 2 * n_touched_vis),
        "bin": dict(flops=0, trans=0, bytes=BIN_BYTES_PER_GAUSSIAN * n),
        "sort": dict(flops=0, trans=0,
                     bytes=SORT_BYTES_PER_PAIR * npairs + SORT_BYTES_PER_TILE * cam.num_tiles),
        "fwd": dict(work["fwd"], trans=hits),
        "bwd": dict(work["bwd"], trans=2 * hits),
    }
    stage_lines = {}
    for s_name, sw in stage_work.items():
        parts = {"fp32": sw["flops"] / (PEAK_FP32_TFLOPS * 1e12),
                 "trans": sw["trans"] / (PEAK_TRANS_GPS * 1e9),
                 "hbm": sw["bytes"] / (PEAK_HBM_GBS * 1e9)}
        bound = max(parts, key=parts.get)
        v = per[s_name]
        stage_lines[s_name] = {
            "ms": round(float(np.median(v)), 4), "ms_p10": round(float(np.percentile(v, 10)), 4),
            "ms_p90": round(float(np.percentile(v, 90)), 4), "ms_min": round(float(np.min(v)), 4),
            "pairs_per_s": round(npairs / (float(np.median(v)) * 1e-3), 1),
            "bytes": sw["bytes"], "flops": sw["flops"], "transcendentals": sw["trans"],
            "bound": bound, "t_roof_ms": round(parts[bound] * 1e3, 4),
            "roofline_frac": round(parts[bound] / (float(np.median(v)) * 1e-3), 4)}
    ms_fwd_total = ms["bin"] + ms["sort"] + ms["fwd"]

    views = None if args.views < 2 else views_stage(args, sc, gsr, dev, means, ls, qs, op, sh)

    cpu = None if args.no_cpu_baseline else cpu_baseline(sc, npairs)

    # every configuration (the headline one from the frames above), with the
    # oracle's knife-edge count and exact hit counts beside it when the CPU leg runs
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    head = frame_diagnostics(gsr, sc, r, n, cus)
    head.update(workload=f"{sc.name}: {n} Gaussians, SH degree {sc.sh_degree}, "
                         f"{cam.width}x{cam.height} image",
                ms_per_step=round(ms_step, 4), ms={k: round(ms[k], 4) for k in stages},
                tile_pairs_per_s=round(npairs / (ms_step * 1e-3), 1),
                raster_roofline_frac=round(raster_frac, 4))
    configs = {str(args.config): head}
    if not args.no_cpu_baseline:
        head["oracle"] = oracle_frame_counts(sc)
    if not args.no_configs:
        del r
        torch.cuda.empty_cache()
        for cfg in (1, 2, 3, 4, 5):
            if cfg == args.config:
                continue
            print(f"[bench] configuration {cfg}", file=sys.stderr, flush=True)
            sc_c, diag = config_line(gsr, dev, cfg, args, cus)
            if not args.no_cpu_baseline:
                diag["oracle"] = oracle_frame_counts(sc_c)
            configs[str(cfg)] = diag
            del sc_c

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
                   "pairs": npairs, "hits": hits, "lane_evaluations": lane_evals,
                   "subtile_hits": sub_hits, "chunk_mode": args.chunk_mode,
                   "chunked_tiles": chunked, "chunks_per_tile": chunks,
                   "schedule": "built inside the sort" if plan_in_sort
                   else "built beside the sort on a second stream"},
        "ms": {k: round(v, 4) for k, v in ms.items()},
        "ms_min": {k: round(v, 4) for k, v in ms_min.items()},
        "ms_project": round(ms_project, 4),
        "ms_project_bwd": round(ms_project_bwd, 4),
        "ms_raster_fwd_bwd": round(ms_raster, 4),
        "ms_kernels": {f"k_render_{k}": round(v, 4) for k, v in kernel_ms.items()},
        "raster_pairs_per_s": round(npairs / (ms_raster * 1e-3), 1),
        "raster_roofline_frac": round(raster_frac, 4),
        "ms_fwd": round(ms_fwd_total, 4), "ms_bwd": round(ms["bwd"], 4),
        "ms_fwd_bwd": round(ms_fwd_total + ms["bwd"], 4),
        "ms_frame": round(ms_project + ms_fwd_total + ms["bwd"], 4),
        "n_visible": n_vis, "n_touched": n_touched, "n_touched_visible": n_touched_vis,
        "stages": stage_lines,
        "views": views,
        "configs": configs,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
