"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Each stage is fed the oracle's own upstream output (stage isolation), so a
rounding difference in one stage cannot change the decisions of the next:
  projection     tolerance (fp32 vs the oracle's fp64)
  binning        offsets, keys, ids bit-exact
  sort, ranges   sorted keys, ids and tile ranges bit-exact
  forward        rgb and T within 1e-5 (2e-4 on knife-edge pixels); last and the
                 number of splats each pixel blended exact away from knife
                 edges; the contributor record (which entries blended into
                 which quarter of their tile) exact away from knife edges
  backward       relative L2 per gradient column <= 1e-3 against the fp64 truth
The end-to-end chain (GPU projection onward) is checked loosely.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import scenegen

pytestmark = pytest.mark.gpu

FWD_TOL, KNIFE_TOL, GRAD_RTOL = 1e-5, 2e-4, 1e-3


def _gsr():
    import gaussian_splatting_differentiable_amd as gsr
    gsr.lib()
    return gsr


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


_REF_CACHE = {}


def reference(cfg):
    if cfg not in _REF_CACHE:
        sc = scenegen.make_config(cfg)
        _REF_CACHE.clear()
        _REF_CACHE[cfg] = (sc, oracle.frame(sc))
    return _REF_CACHE[cfg]


def check_projection(sc, ref_splats, gpu_splats):
    vis = ref_splats[:, 9] > 0
    gvis = gpu_splats[:, 9] > 0
    knife = np.abs(ref_splats[:, 9]) < 1e-4
    assert np.array_equal(vis[~knife], gvis[~knife])
    both = vis & gvis
    r, g = ref_splats[both].astype(np.float64), gpu_splats[both].astype(np.float64)
    # conic entries share a per-splat scale sqrt(a c); colours an absolute floor
    conic_scale = np.sqrt(r[:, 2] * r[:, 4])[:, None]
    tol = 1e-5 * np.abs(r)
    tol[:, [0, 1, 10]] += 1e-6 * np.abs(r[:, [0, 1, 10]]).max(axis=0)
    tol[:, 2:5] += 1e-5 * conic_scale
    tol[:, 5] += 1e-7
    tol[:, 6:9] += 1e-5
    tol[:, 9] += 1e-6
    bad = np.abs(g - r) > tol
    assert not bad.any(), (np.nonzero(bad.any(axis=1))[0][:5], np.nonzero(bad.any(axis=0))[0])
    assert np.all(gpu_splats[~gvis][:, 9] == -1) and np.all(gpu_splats[~gvis][:, [0, 1, 2, 5, 10]] == 0)


def run_stages(gsr, sc, ref, capacity=None, sched=None, background=None, dL_dT=None):
    """GPU bin/sort/fwd/bwd fed the oracle's splats. Returns host arrays.
    background / dL_dT (host arrays) select gs_render_fwd_bg / gs_render_bwd_bg."""
    cam = sc.camera
    n = sc.n
    npairs = len(ref["sorted_ids"])
    cap = capacity if capacity is not None else max(npairs, 1)
    r = gsr.Rasterizer(cam, capacity=cap, sched=sched)
    r._ensure(n, cap)
    r.splats[:n].copy_(dev(ref["splats"]))
    I = r.bin_and_sort(n, want_keys=True, want_emission=True)
    out = dict(I=I, offsets=host(r.offsets), keys=host(r.keys)[:I].view(np.uint64),
               ids=host(r.ids)[:I], sorted_keys=host(r.sorted_keys)[:I].view(np.uint64),
               sorted_ids=host(r.sorted_ids)[:I], ranges=host(r.ranges))
    # forward/backward on the oracle's sorted list (stage isolation); the state is
    # cleared so that contributor words the forward does not write read as zero
    r.sorted_ids[:npairs].copy_(dev(ref["sorted_ids"]))
    r.ranges.copy_(dev(ref["ranges"]))
    r.clear_state()
    r.render_fwd(n, stats=True, background=background)
    out["contrib"] = read_contrib(r, ref["ranges"])
    grads = r.render_bwd(n, dev(sc.dL_drgb), background=background,
                         dL_dT=None if dL_dT is None else dev(dL_dT))
    r.check("stage parity frame")
    out.update(rgb=host(r.rgb), T=host(r.T), last=host(r.last), grads=host(grads),
               stats=host(r.stats), pixel_hits=host(r.pixel_hits), plan=read_plan(r),
               bwd_queue=read_bwd_queue(r), tiles=r.tiles)
    return out


def check_binning(ref, out):
    assert out["I"] == len(ref["ids"])
    assert np.array_equal(out["offsets"].astype(np.int64), ref["offsets"])
    assert np.array_equal(out["keys"], ref["keys"])
    assert np.array_equal(out["ids"], ref["ids"])


def check_sort(ref, out):
    assert np.array_equal(out["sorted_keys"], ref["sorted_keys"])
    assert np.array_equal(out["sorted_ids"], ref["sorted_ids"])
    assert np.array_equal(out["ranges"], ref["ranges"])


def check_forward(ref, out):
    f = ref["fwd"]
    knife = f["knife"]
    d_rgb = np.abs(out["rgb"] - f["rgb"]).max(axis=0)
    d_T = np.abs(out["T"] - f["T"])
    assert d_rgb[~knife].max(initial=0) <= FWD_TOL, d_rgb[~knife].max()
    assert d_T[~knife].max(initial=0) <= FWD_TOL, d_T[~knife].max()
    assert d_rgb[knife].max(initial=0) <= KNIFE_TOL and d_T[knife].max(initial=0) <= KNIFE_TOL
    assert np.array_equal(out["last"][~knife], f["last"][~knife])
    # every pixel blended exactly the oracle's splats (a dropped or extra hit of
    # any depth shows here, however small its colour)
    ph = out["pixel_hits"]
    bad = (ph != f["pixel_hits"]) & ~knife
    assert not bad.any(), (np.argwhere(bad)[:5], int(bad.sum()))
    assert int(out["stats"][0]) == int(ph.sum())
    if "contrib" in out:
        check_contrib(ref, out["contrib"])


def check_contrib(ref, contrib):
    """The forward's contributor record equals the oracle's per-quarter hits of
    every list entry, except in quarters that hold a knife-edge pixel."""
    f = ref["fwd"]
    H, W = f["T"].shape
    tx = (W + 15) // 16
    ranges = ref["ranges"]
    knife_q = np.zeros(len(ranges) * 4, bool)
    ky, kx = np.nonzero(f["knife"])
    knife_q[((ky // 16) * tx + kx // 16) * 4 + ((kx % 16) // 8) + 2 * ((ky % 16) // 8)] = True
    tile_of = np.repeat(np.arange(len(ranges)), ranges[:, 1] - ranges[:, 0])
    pq = f["pair_quarters"]
    for q in range(4):
        exp = (pq >> q) & 1
        got = contrib[q]
        ok = knife_q[tile_of * 4 + q] | (exp == got)
        assert ok.all(), (q, np.nonzero(~ok)[0][:5], int((~ok).sum()))


def check_backward(ref, out):
    g, gref = out["grads"].astype(np.float64), ref["grads"]
    num = np.linalg.norm(g - gref, axis=0)
    den = np.linalg.norm(gref, axis=0)
    rel = num / np.maximum(den, 1e-30)
    assert np.all(rel <= GRAD_RTOL), rel


@pytest.mark.parametrize("cfg", [1, 2])
def test_projection_parity(cfg):
    gsr = _gsr()
    sc, ref = reference(cfg)
    r = gsr.Rasterizer(sc.camera, capacity=16)
    sp = r.project(dev(sc.means), dev(sc.log_scales), dev(sc.quats), dev(sc.opacities), dev(sc.sh),
                   sc.sh_degree)
    check_projection(sc, ref["splats"], host(sp))


@pytest.mark.parametrize("cfg", [1, 2])
def test_stage_parity(cfg):
    gsr = _gsr()
    sc, ref = reference(cfg)
    out = run_stages(gsr, sc, ref)
    check_binning(ref, out)
    check_sort(ref, out)
    check_forward(ref, out)
    check_backward(ref, out)


@pytest.mark.parametrize("seed,W,H,n", [(101, 83, 45, 2000), (102, 17, 70, 900), (103, 200, 33, 5000)])
def test_ragged_scenes(seed, W, H, n):
    gsr = _gsr()
    sc = scenegen.random_scene(seed, n, W, H, 0.9 * W, degree=2, log_scale=(-2.0, 0.6),
                               opacity=(1.0, 2.0))
    ref = oracle.frame(sc)
    out = run_stages(gsr, sc, ref)
    check_binning(ref, out)
    check_sort(ref, out)
    check_forward(ref, out)
    check_backward(ref, out)


def test_large_splats_sort_matches_oracle():
    """Splats covering several tile rows each (about seven on average): the
    pairs the sort generates row by row, their order and the tile ranges are
    the oracle's, bit for bit."""
    gsr = _gsr()
    sc = scenegen.random_scene(104, 2000, 160, 150, 150.0, degree=1, log_scale=(-0.7, 0.3),
                               opacity=(1.0, 1.0))
    ref = oracle.frame(sc, fwd=False)
    vis = np.diff(ref["offsets"]) > 0
    tiles_x = (sc.camera.width + 15) // 16
    ty = (ref["keys"] >> np.uint64(32)).astype(np.int64) // tiles_x
    rows = len(np.unique(ref["ids"].astype(np.int64) * 4096 + ty))
    assert rows > 5 * vis.sum()
    cam = sc.camera
    r = gsr.Rasterizer(cam, capacity=len(ref["sorted_ids"]))
    r._ensure(sc.n, len(ref["sorted_ids"]))
    r.splats[:sc.n].copy_(dev(ref["splats"]))
    I = r.bin_and_sort(sc.n, want_keys=True)
    assert I == len(ref["sorted_ids"])
    assert np.array_equal(host(r.sorted_keys)[:I].view(np.uint64), ref["sorted_keys"])
    assert np.array_equal(host(r.sorted_ids)[:I], ref["sorted_ids"])
    assert np.array_equal(host(r.ranges), ref["ranges"])


def test_depth_range_beyond_sixteen_exponents_sorts_exactly():
    """Depths from about 0.3 to about 30,000: the keys' fp32 exponents span 16
    values or more, so the depth sort needs its fourth pass (bits 27-31 of the
    key less the smallest exponent). Half of the splats are moved 10^4 times
    farther, with positions and scales grown alike so that they stay on screen."""
    gsr = _gsr()
    sc = scenegen.random_scene(107, 3000, 150, 110, 150.0, depth=(0.3, 3.0),
                               log_scale=(-2.5, 0.3))
    far = np.arange(sc.n) % 2 == 1
    sc.means[far] *= np.float32(1.0e4)
    sc.log_scales[far] += np.float32(np.log(1.0e4))
    ref = oracle.frame(sc, fwd=False)
    vis = np.diff(ref["offsets"]) > 0
    e = (ref["splats"][vis, 10].view(np.uint32) >> np.uint32(23)) & np.uint32(255)
    assert int(e.max()) - int(e.min()) >= 16, (int(e.min()), int(e.max()))
    r = gsr.Rasterizer(sc.camera, capacity=len(ref["sorted_ids"]))
    r._ensure(sc.n, len(ref["sorted_ids"]))
    r.splats[:sc.n].copy_(dev(ref["splats"]))
    I = r.bin_and_sort(sc.n, want_keys=True)
    assert I == len(ref["sorted_ids"])
    assert np.array_equal(host(r.sorted_keys)[:I].view(np.uint64), ref["sorted_keys"])
    assert np.array_equal(host(r.sorted_ids)[:I], ref["sorted_ids"])
    assert np.array_equal(host(r.ranges), ref["ranges"])


@pytest.mark.parametrize("w,h", [(700, 500), (1600, 1400)])
def test_tile_passes_without_keys_match_with_keys(w, h):
    """The production path writes no sorted keys: its ids and ranges equal the
    oracle's as those of the checking path do, on 1408 tiles (the high tile
    digit ranked on 5 bits) and 8800 (on 8)."""
    gsr = _gsr()
    sc = scenegen.random_scene(w + h, 4000, w, h, 0.9 * w)
    ref = oracle.frame(sc, fwd=False)
    I0 = len(ref["sorted_ids"])
    assert I0 > 0
    for want_keys in (False, True):
        r = gsr.Rasterizer(sc.camera, capacity=I0)
        r._ensure(sc.n, I0)
        r.splats[:sc.n].copy_(dev(ref["splats"]))
        r.sorted_ids.fill_(-1)
        I = r.bin_and_sort(sc.n, want_keys=want_keys)
        assert I == I0
        assert np.array_equal(host(r.sorted_ids)[:I], ref["sorted_ids"]), want_keys
        assert np.array_equal(host(r.ranges), ref["ranges"]), want_keys


def test_capacity_overflow_reports_and_recovers():
    gsr = _gsr()
    sc, ref = reference(1)
    npairs = len(ref["sorted_ids"])
    r = gsr.Rasterizer(sc.camera, capacity=16)
    r._ensure(sc.n, 16)
    r.splats[:sc.n].copy_(dev(ref["splats"]))
    r.ranges.fill_(-7)
    r.rgb.fill_(5.0)
    gsr.gs_bin_tiles(sc.n, r.splats, r.cam, 16, r.offsets, r.keys, r.ids, r.status, r.workspace)
    gsr.gs_sort_keys(sc.n, r.splats, r.offsets, 16, r.cam, None, r.sorted_ids, r.ranges,
                     r.status, r.workspace)
    r.render_fwd(sc.n)
    g = r.render_bwd(sc.n, dev(sc.dL_drgb))
    st, I = r.frame_status(sc.n)                  # read once, after the frame
    assert st == gsr.GS_ERR_CAPACITY and I == npairs
    assert np.all(host(r.ranges) == 0)          # later calls do nothing for the frame
    assert np.all(host(r.rgb) == 5.0)           # the forward did not run
    assert np.all(host(g) == 0)                 # the backward only zeroed its output
    I = r.run_frame(sc.n, dev(sc.dL_drgb))        # the driver grows and re-runs
    assert I == npairs and r.capacity >= npairs
    assert np.array_equal(host(r.sorted_ids)[:I], ref["sorted_ids"])


def test_empty_and_all_culled():
    gsr = _gsr()
    cam = scenegen.pinhole(40, 24, 30.0)
    sc = scenegen.random_scene(7, 50, 40, 24, 30.0)
    sc.means[:, 2] = -1.0                        # everything behind the camera
    ref = oracle.frame(sc)
    assert len(ref["sorted_ids"]) == 0
    out = run_stages(gsr, sc, ref, capacity=8)
    assert out["I"] == 0 and np.all(out["ranges"] == 0)
    assert np.all(out["rgb"] == 0) and np.all(out["T"] == 1) and np.all(out["grads"] == 0)


def test_end_to_end_chain_small():
    """GPU projection onward; pair counts may differ by boundary splats only."""
    gsr = _gsr()
    sc, ref = reference(2)
    r = gsr.Rasterizer(sc.camera, capacity=len(ref["sorted_ids"]) + 4096)
    n = sc.n
    r.project(dev(sc.means), dev(sc.log_scales), dev(sc.quats), dev(sc.opacities), dev(sc.sh),
              sc.sh_degree)
    I = r.bin_and_sort(n)
    r.render_fwd(n)
    g = host(r.render_bwd(n, dev(sc.dL_drgb))).astype(np.float64)
    assert abs(I - len(ref["sorted_ids"])) <= 1e-4 * I + 4
    d = np.abs(host(r.rgb) - ref["fwd"]["rgb"]).max(axis=0)
    assert np.quantile(d, 0.999) < 1e-4
    rel = np.linalg.norm(g - ref["grads"], axis=0) / np.linalg.norm(ref["grads"], axis=0)
    assert np.all(rel < 1e-2), rel


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_full_size_configs(cfg):
    """Full-size scenes: every stage against the oracle over the whole frame."""
    gsr = _gsr()
    sc, ref = reference(cfg)
    r = gsr.Rasterizer(sc.camera, capacity=16)
    sp = r.project(dev(sc.means), dev(sc.log_scales), dev(sc.quats), dev(sc.opacities), dev(sc.sh),
                   sc.sh_degree)
    check_projection(sc, ref["splats"], host(sp))
    del r
    out = run_stages(gsr, sc, ref)
    check_binning(ref, out)
    check_sort(ref, out)
    check_forward(ref, out)
    check_backward(ref, out)
    if cfg == 5:
        assert int(out["stats"][3]) >= 1   # the policy chunks urban's heaviest tiles
    print(f"config {cfg}: pairs {out['I']}, hits {int(out['stats'][0])}, chunked tiles "
          f"{int(out['stats'][3])}, knife-edge pixels {int(ref['fwd']['knife'].sum())}",
          flush=True)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_backward_pieces_between_cuts(cfg):
    """In a frame with few tiles (tiny, small), long quarter walks are
    differentiated as pieces between cuts, side by side, each from the forward
    pass's state at its cut; garden (whole tiles) walks every tile whole. The
    backward queue serves every walk once, and the gradients match the oracle
    element by element."""
    gsr = _gsr()
    sc, ref = reference(cfg)
    out = run_stages(gsr, sc, ref)
    check_forward(ref, out)
    check_backward(ref, out)
    check_backward_elementwise(ref, out)
    quarters = 2 * out["tiles"] < 4 * _workers()
    assert quarters == (cfg != 3)
    npieces = check_bwd_queue(*out["bwd_queue"], ref["ranges"], quarters)
    assert npieces >= {1: 10, 2: 500, 3: 0}[cfg], npieces
    print(f"config {cfg}: walks in pieces {npieces}", flush=True)


def test_frame_of_more_than_8192_tiles():
    """A 1600x1400 frame with a ragged last row and column (8800 tiles): the
    schedule keeps its working arrays in the forward state instead of LDS, and
    every stage still matches the oracle."""
    gsr = _gsr()
    sc = scenegen.random_scene(105, 120_000, 1601, 1399, 1400.0, degree=1,
                               log_scale=(-3.0, 0.6), opacity=(0.5, 1.5))
    assert sc.camera.num_tiles > 8192
    ref = oracle.frame(sc)
    out = run_stages(gsr, sc, ref)
    check_binning(ref, out)
    check_sort(ref, out)
    check_forward(ref, out)
    check_backward(ref, out)
    check_queues(out["plan"], (sc.camera.width + 15) // 16)


def test_sort_rejects_a_workspace_without_its_binning_pass():
    """The binning pass tags the workspace with its sizes and the sort uses the
    tag up: a second sort of the same frame, or a sort whose sizes differ from
    the binning pass's, reports GS_ERR_WORKSPACE through the status word and
    leaves empty ranges."""
    gsr = _gsr()
    sc, ref = reference(1)
    n, npairs = sc.n, len(ref["sorted_ids"])
    r = gsr.Rasterizer(sc.camera, capacity=npairs + 64)
    r._ensure(n, npairs + 64)
    r.splats[:n].copy_(dev(ref["splats"]))
    assert r.bin_and_sort(n) == npairs
    gsr.gs_sort_keys(n, r.splats, r.offsets, r.capacity, r.cam, None, r.sorted_ids, r.ranges,
                     r.status, r.workspace)
    assert r.frame_status(n)[0] == gsr.GS_ERR_WORKSPACE
    assert np.all(host(r.ranges) == 0)
    # sizes that differ from the binning pass's: n - 1 splats
    gsr.gs_bin_tiles(n, r.splats, r.cam, r.capacity, r.offsets, None, None, r.status, r.workspace)
    gsr.gs_sort_keys(n - 1, r.splats, r.offsets, r.capacity, r.cam, None, r.sorted_ids, r.ranges,
                     r.status, r.workspace)
    assert r.frame_status(n)[0] == gsr.GS_ERR_WORKSPACE
    # an error is never overwritten by the later calls of the frame
    r.render_fwd(n)
    r.render_bwd(n, dev(sc.dL_drgb))
    assert r.frame_status(n)[0] == gsr.GS_ERR_WORKSPACE
    # and the next frame starts clean
    assert r.run_frame(n, dev(sc.dL_drgb)) == npairs


def test_state_too_small_for_the_frame_is_reported():
    """A forward state sized for fewer pairs than the frame holds: the schedule
    reports GS_ERR_WORKSPACE and neither raster kernel runs."""
    gsr = _gsr()
    sc, ref = reference(1)
    n, npairs = sc.n, len(ref["sorted_ids"])
    r = gsr.Rasterizer(sc.camera, capacity=npairs)
    r._ensure(n, npairs)
    r.splats[:n].copy_(dev(ref["splats"]))
    assert r.bin_and_sort(n) == npairs
    small = torch.empty(gsr.fwd_state_size(sc.camera.width, sc.camera.height, 0),
                        dtype=torch.uint8, device="cuda")
    r.fwd_state = small
    r.rgb.fill_(3.0)
    r.render_fwd(n)
    g = r.render_bwd(n, dev(sc.dL_drgb))
    assert r.frame_status(n)[0] == gsr.GS_ERR_WORKSPACE
    assert np.all(host(r.rgb) == 3.0) and np.all(host(g) == 0)


# ---------------------------------------------------------------- scheduling and chunking

def _plan_layout(T):
    """Offsets into the opaque forward state, read here for checking only:
    header (h, k, nA, nplain, err, ntiles, group offsets, pass-A counts, static
    hand-out counts, ...), queue heads, per-quarter bounds, LPT order, sorted
    counts, the queue items, ..., the backward's items (up to 4 per forward
    item), the cut records, the contributor words (last)."""
    rnd = lambda b: (b + 255) // 256 * 256
    cq = 4096 * 4
    hdr = 0
    heads = rnd(208)
    sub_last = heads + rnd(4 * 2 * 8 * 16)
    order = sub_last + rnd(16 * T)
    counts = order + rnd(4 * T)
    items = counts + rnd(4 * T)
    off = items + rnd(4 * (4 * T + 2 * cq))
    for b in (4 * 2048 * 4, 4 * cq, 4 * 2048 * 4, 4 * cq, 4 * cq * 64, 4 * cq * 64 * 3,
              4 * cq * 64, 4 * cq * 64, 4 * cq * 64):
        off += rnd(b)
    bitems = off
    qcut = bitems + rnd(4 * 4 * (4 * T + 2 * cq))
    tlen = qcut + rnd(4 * 4 * T) + rnd(4 * (T if T <= 2048 else 0) * 15 * 256)
    bcnt = tlen + rnd(8 * T)
    blist = bcnt + rnd(4 * 8 * 64)
    off = blist + rnd(4 * 64 * (4 * T + 2 * cq))
    return dict(hdr=hdr, heads=heads, sub_last=sub_last, order=order, counts=counts, items=items,
                bitems=bitems, qcut=qcut, bcnt=bcnt, blist=blist, contrib=off)


def read_contrib(r, ranges):
    """The forward's contributor record as one 0/1 array per quarter over the
    list positions: quarter q's word for tile t and batch m is word
    (start_t >> 6) + t + m of array q (nw words each, from the header)."""
    T = r.tiles
    L = _plan_layout(T)
    raw = host(r.fwd_state)
    nw = int(raw[200:208].view(np.int64)[0])
    assert nw >= r.capacity // 64 + T + 2
    words = raw[L["contrib"]:L["contrib"] + 8 * 4 * nw].view(np.uint64).reshape(4, nw)
    npairs = int(ranges[-1, 1]) if len(ranges) else 0
    out = np.zeros((4, npairs), np.uint8)
    for t in range(T):
        s, e = int(ranges[t, 0]), int(ranges[t, 1])
        if e == s:
            continue
        k = np.arange(e - s)
        w = words[:, (s >> 6) + t + (k >> 6)]
        out[:, s:e] = ((w >> (k & 63).astype(np.uint64)) & np.uint64(1)).astype(np.uint8)
    return out


def read_plan(r):
    T = r.tiles
    L = _plan_layout(T)
    raw = host(r.fwd_state)
    hdr = raw[L["hdr"]:L["hdr"] + 208].view(np.int32)
    order = raw[L["order"]:L["order"] + 4 * T].view(np.int32)
    counts = raw[L["counts"]:L["counts"] + 4 * T].view(np.int32)
    qoff = hdr[6:15].copy()
    items = raw[L["items"]:L["items"] + 4 * int(qoff[-1])].view(np.int32)
    assert int(hdr[5]) == T
    return dict(h=int(hdr[0]), k=int(hdr[1]), nA=int(hdr[2]), err=int(hdr[4]), order=order,
                counts=counts, qoff=qoff, qa=hdr[15:23].copy(), items=items.copy(),
                run_f=int(hdr[47]))


CUT_BATCHES = (2, 4, 8)  # a plain walk's cut points, in 64-entry batches


def read_bwd_queue(r):
    """The backward's items per group, and per quarter the forward's walk
    length (1 + the last entry any pixel blended) and the cuts it reached.
    A frame with few tiles has them in the preparation's list; any other frame
    in the bins the forward filed them in (group g, bin b: the b-th of 64
    quarter-octave bins of the walk length, longest first), read in bin order,
    and for those the bins are returned as well."""
    T = r.tiles
    L = _plan_layout(T)
    raw = host(r.fwd_state)
    hdr = raw[:256].view(np.int32)
    qoff, qa, nb, bmode = hdr[6:15], hdr[15:23], hdr[39:47], int(hdr[61])
    groups, bins = [], []
    if bmode:
        bcnt = raw[L["bcnt"]:L["bcnt"] + 4 * 8 * 64].view(np.int32).reshape(8, 64)
        for g in range(8):
            span = int(qoff[g + 1]) - int(qoff[g])
            its, bs = [], []
            for b in range(64):
                base = L["blist"] + 4 * (64 * int(qoff[g]) + b * span)
                its.append(raw[base:base + 4 * int(bcnt[g, b])].view(np.int32))
                bs.append(np.full(int(bcnt[g, b]), b))
            groups.append(np.concatenate(its).copy())
            bins.append(np.concatenate(bs))
    else:
        for g in range(8):
            base = L["bitems"] + 4 * 4 * (int(qoff[g]) + int(qa[g]))
            groups.append(raw[base:base + 4 * int(nb[g])].view(np.int32).copy())
    sub_last = raw[L["sub_last"]:L["sub_last"] + 16 * T].view(np.int32).reshape(T, 4).copy()
    qcut = raw[L["qcut"]:L["qcut"] + 16 * T].view(np.int32).reshape(T, 4).copy()
    return groups, sub_last, qcut, (bins if bmode else None)


def check_bwd_queue(groups, sub_last, qcut, bins, ranges, quarters):
    """Every plain tile's walk (or, when quarters, every quarter's) is served
    once: whole, or as all of its pieces between the cuts below its length;
    a quarter reached every cut below its walk's end and none past its list.
    Only a frame walked by quarters (few tiles) records cuts. Items filed in
    bins by the forward: a plain item's bin is that of its walk length (64
    quarter-octave bins, longest first; the device's log2 may round a length
    at a bin edge either way)."""
    items = np.concatenate(groups)
    kind, quad, p, idx = (items >> 30) & 3, (items >> 28) & 3, (items >> 24) & 15, items & 0xFFFFFF
    assert not np.any(kind == 1)
    if bins is not None:
        b = np.concatenate(bins)
        pl = kind != 2
        walk = np.where(kind[pl] == 3, sub_last[idx[pl], quad[pl]], sub_last[idx[pl]].max(axis=1))
        l4 = 4.0 * np.log2(np.maximum(walk, 0) + 1.0)
        want = 63 - np.minimum(np.floor(l4), 63)
        edge = np.abs(l4 - np.round(l4)) < 1e-3
        assert np.all((b[pl] == want) | (edge & (np.abs(b[pl] - want) <= 1)))
    plain = kind != 2
    seen = {}
    for kd, q, pp, t in zip(kind[plain], quad[plain], p[plain], idx[plain]):
        key = (int(t), int(q) if kd == 3 else -1)
        # by quarters: every tile of a frame with few tiles; in any other frame
        # the tiles whose whole walk spans more than 2048 entries
        assert (kd == 3) == (quarters or int(sub_last[t].max()) > 2048)
        seen.setdefault(key, []).append(int(pp))
    T = len(ranges)
    h = len(set(int(s) for s in idx[kind == 2]))  # chunked tiles (their slots)
    nsplit = sum(1 for (t, q) in seen if q >= 0) // 4
    assert len(seen) == (4 * (T - h) if quarters else T - h + 3 * nsplit)
    npieces = 0
    for (t, q), ps in seen.items():
        walk = int(sub_last[t, q]) if q >= 0 else int(sub_last[t].max())
        nb = (max(walk, 0) + 63) // 64
        want = 1 + sum(c < nb for c in CUT_BATCHES)
        assert sorted(ps) in ([0], list(range(1, want + 1))), (t, q, ps, nb)
        npieces += len(ps) > 1
    if not quarters:
        assert npieces == 0 and not qcut.any()
        return npieces
    n_t = ranges[:, 1] - ranges[:, 0]
    for c, b in enumerate(CUT_BATCHES):
        assert np.all((qcut > c) >= (sub_last > 64 * b))
        assert np.all((qcut > c) <= (n_t[:, None] > 64 * b))
    return npieces


def check_backward_elementwise(ref, out):
    """Per gradient element: 99.9% within 5e-4 of |ref| + 1e-3 rms (the
    component's), where the norm-wise check could hide a few bad splats. A
    gradient is a sum over many pixels of terms of both signs, so fp32 leaves
    up to a few 1e-4 on the worst of a thousand splats; a wrong term is off by
    far more."""
    g, gref = out["grads"].astype(np.float64), ref["grads"]
    rms = np.sqrt((gref ** 2).mean(axis=0))
    e = np.abs(g - gref) / (np.abs(gref) + 1e-3 * rms)
    q = np.quantile(e, 0.999, axis=0)
    assert np.all(q <= 5e-4), q
    assert np.all(e.max(axis=0) <= 0.2), e.max(axis=0)


def check_queues(plan, tiles_x):
    """Group g's queue: the pass-A items of its chunked tiles, as many pass-B
    items, then the quarters of its other tiles in longest-first order; every
    item exactly once, every tile in the group of its image strip."""
    h, k, order, items, qoff = plan["h"], plan["k"], plan["order"], plan["items"], plan["qoff"]
    T = len(order)
    group = lambda tile: (tile % tiles_x) * 8 // tiles_x
    kind, quad, p, idx = (items >> 30) & 3, (items >> 28) & 3, (items >> 24) & 15, items & 0xFFFFFF
    rank = np.empty(T, np.int64)
    rank[order] = np.arange(T)
    seen_a, seen_b, seen_p = set(), set(), set()
    for g in range(8):
        lo, hi, qa = int(qoff[g]), int(qoff[g + 1]), int(plan["qa"][g])
        assert np.all(kind[lo:lo + qa] == 1) and np.all(kind[lo + qa:lo + 2 * qa] == 2)
        assert np.all(kind[lo + 2 * qa:hi] == 0)
        for a, b in ((lo, lo + qa), (lo + qa, lo + 2 * qa)):
            slots = idx[a:b]
            assert np.all(slots < h) and all(group(order[s]) == g for s in slots)
            assert np.all(np.diff(slots) >= 0)  # chunked tiles in LPT order
        for i in range(lo, lo + qa):
            seen_a.add((int(idx[i]), int(p[i]), int(quad[i])))
        for i in range(lo + qa, lo + 2 * qa):
            seen_b.add((int(idx[i]), int(p[i]), int(quad[i])))
        tiles = idx[lo + 2 * qa:hi]
        assert all(group(t) == g for t in tiles)
        assert np.all(np.diff(rank[tiles]) >= 0)  # longest first, quarters of a tile together
        assert np.all(rank[tiles] >= h)
        for i in range(lo + 2 * qa, hi):
            seen_p.add((int(idx[i]), int(quad[i])))
    assert len(seen_a) == len(seen_b) == 4 * h * (k if h else 0)
    assert seen_a == seen_b and all(pp < k for _, pp, _ in seen_a)
    assert len(seen_p) == 4 * (T - h) and int(qoff[-1]) == 8 * h * k + 4 * (T - h)


def _workers():
    """K of the policy: the library's persistent worker waves (16 per CU), four per tile."""
    return torch.cuda.get_device_properties(0).multi_processor_count * 16 / 4.0


@pytest.mark.parametrize("k", [2, 4, 8, 16])
def test_forced_chunking_matches_oracle(k):
    """Every tile split into k depth chunks: exact composition, so the results
    still match the unchunked oracle to the same bars."""
    gsr = _gsr()
    sc, ref = reference(2)
    sched = gsr.make_sched(chunk_mode=2, force_k=k, force_h=0)
    out = run_stages(gsr, sc, ref, sched=sched)
    check_forward(ref, out)
    check_backward(ref, out)
    assert int(out["stats"][3]) == min(sc.camera.num_tiles, gsr.HK_MAX // k)
    check_queues(out["plan"], (sc.camera.width + 15) // 16)


@pytest.mark.parametrize("k,h", [(2, 3), (16, 40)])
def test_forced_chunking_ragged(k, h):
    gsr = _gsr()
    sc = scenegen.random_scene(104, 6000, 150, 70, 120.0, degree=1, log_scale=(-2.2, 0.7),
                               opacity=(1.0, 2.0))
    ref = oracle.frame(sc)
    out = run_stages(gsr, sc, ref, sched=gsr.make_sched(chunk_mode=2, force_k=k, force_h=h))
    check_forward(ref, out)
    check_backward(ref, out)
    assert out["plan"]["h"] == h and out["plan"]["k"] == k
    check_queues(out["plan"], (sc.camera.width + 15) // 16)


def _policy_frame(gsr, counts, W, H):
    """Run the device schedule on given tile counts (a dummy list of culled splats)."""
    cam = scenegen.pinhole(W, H, float(W))
    T = cam.num_tiles
    assert len(counts) == T
    ranges = np.zeros((T, 2), np.int32)
    ranges[:, 1] = np.cumsum(counts)
    ranges[1:, 0] = ranges[:-1, 1]
    I = int(ranges[-1, 1])
    r = gsr.Rasterizer(cam, capacity=max(I, 1))
    r._ensure(1, max(I, 1))
    r.splats.zero_()
    r.splats[:, 9] = -1.0
    r.sorted_ids.zero_()
    r.ranges.copy_(dev(ranges))
    r.render_fwd(1)
    return read_plan(r)


@pytest.mark.parametrize("case", ["pareto", "one_outlier", "flat", "two_level"])
@pytest.mark.parametrize("W,H", [(1920, 1080), (3840, 2160)])  # 8160 tiles (LDS path), 32400
def test_device_policy_equals_host_policy(case, W, H):
    gsr = _gsr()
    rng = np.random.default_rng({"pareto": 1, "one_outlier": 2, "flat": 3, "two_level": 4}[case])
    T = ((W + 15) // 16) * ((H + 15) // 16)
    if case == "pareto":
        counts = (rng.pareto(1.2, T) * 300).astype(np.int64)
    elif case == "one_outlier":
        counts = rng.integers(50, 400, T)
        counts[1234 % T] = 250_000
    elif case == "flat":
        counts = np.full(T, 700)
    else:
        counts = np.where(rng.random(T) < 0.02, 40_000, 900)
    counts = np.minimum(counts, 2_000_000).astype(np.int32)
    plan = _policy_frame(gsr, counts, W, H)
    assert plan["err"] == 0 and plan["run_f"] == 1
    # exact LPT order: count descending, ties by tile id
    ref_order = np.lexsort((np.arange(T), -counts.astype(np.int64)))
    assert np.array_equal(plan["order"], ref_order)
    assert np.array_equal(plan["counts"], counts[ref_order])
    f32 = lambda v: float(np.float32(v))  # the knobs travel as fp32 in gs_sched
    h, k = oracle.chunk_policy(counts[ref_order], _workers(), f32(gsr.DEFAULT_LAMBDA),
                               f32(gsr.DEFAULT_BETA), f32(gsr.DEFAULT_EPS), gsr.HK_MAX)
    assert (plan["h"], plan["k"] if plan["h"] else 1) == (h, k), (plan["h"], plan["k"], h, k)
    assert plan["nA"] == 4 * h * (k if h else 0)
    assert plan["qoff"][0] == 0 and np.all(np.diff(plan["qoff"]) >= 0)
    check_queues(plan, (W + 15) // 16)
    if case == "one_outlier":
        assert h >= 1
    if case == "flat":
        assert h == 0


def test_forward_without_stats_is_identical():
    """The production forward (no statistics buffer) is a separate instantiation
    of the kernel: it must give the same images, bit for bit, as the counting
    one that the parity tests above check against the oracle, on a chunked and
    an unchunked plan."""
    gsr = _gsr()
    sc, ref = reference(1)
    n, npairs = sc.n, len(ref["sorted_ids"])
    for sched in (None, gsr.make_sched(chunk_mode=2, force_k=4, force_h=6)):
        r = gsr.Rasterizer(sc.camera, capacity=max(npairs, 1), sched=sched)
        r._ensure(n, max(npairs, 1))
        r.splats[:n].copy_(dev(ref["splats"]))
        r.sorted_ids[:npairs].copy_(dev(ref["sorted_ids"]))
        r.ranges.copy_(dev(ref["ranges"]))
        r.render_fwd(n, stats=True)
        a = [host(t).copy() for t in (r.rgb, r.T, r.last)]
        r.render_fwd(n, stats=False)
        b = [host(t) for t in (r.rgb, r.T, r.last)]
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        check_forward(ref, dict(rgb=b[0], T=b[1], last=b[2], stats=host(r.stats),
                                pixel_hits=host(r.pixel_hits)))


def test_kernel_timing_entry_points():
    """gs_timing_start / gs_timing_read record one duration per raster kernel
    launch, in launch order, and stop recording when read."""
    gsr = _gsr()
    sc, ref = reference(1)
    n, npairs = sc.n, len(ref["sorted_ids"])
    r = gsr.Rasterizer(sc.camera, capacity=max(npairs, 1))
    r._ensure(n, max(npairs, 1))
    r.splats[:n].copy_(dev(ref["splats"]))
    r.sorted_ids[:npairs].copy_(dev(ref["sorted_ids"]))
    r.ranges.copy_(dev(ref["ranges"]))
    dL = dev(sc.dL_drgb)
    gsr.gs_timing_start()
    for _ in range(3):
        r.render_fwd(n)
        r.render_bwd(n, dL)
    fwd, bwd = gsr.gs_timing_read(0), gsr.gs_timing_read(1)
    assert len(fwd) == 3 and len(bwd) == 3
    assert all(0.0 < t < 1000.0 for t in fwd + bwd)
    r.render_fwd(n)  # not recorded any more
    assert len(gsr.gs_timing_read(0)) == 3
    with pytest.raises(gsr.GsError):
        gsr.gs_timing_read(2)
