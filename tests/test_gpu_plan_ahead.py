"""The tile schedule built ahead of the forward (gs_plan_tiles, from the
binning pass's per-tile counts, on a second stream beside the sort).

  tile counts    gs_bin_tiles' tile_counts equal the oracle's per-tile pair
                 counts exactly (configs 1 and 2, a batch of views)
  same plan      a plan built ahead equals the one the forward builds itself,
                 field for field, and gives the same images bit for bit
  handed over    the forward uses a plan built ahead even when its order is not
                 the frame's (any plan of the grid gives the same images)
  refused        a plan for another pair total is reported (GS_ERR_WORKSPACE);
                 a plan built with other knobs is rebuilt by the forward; a
                 plan over the state's capacity is reported
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import scenegen
from test_gpu_parity import dev, host, read_plan, check_queues

pytestmark = pytest.mark.gpu


def _gsr():
    import gaussian_splatting_differentiable_amd as gsr
    gsr.lib()
    return gsr


_REF = {}


def reference(cfg):
    if cfg not in _REF:
        sc = scenegen.make_config(cfg)
        _REF[cfg] = (sc, oracle.frame(sc))
    return _REF[cfg]


def rasterizer(gsr, sc, ref, sched=None, plan_ahead=True, cap=None):
    n = sc.n
    cap = cap if cap is not None else max(len(ref["sorted_ids"]), 1)
    r = gsr.Rasterizer(sc.camera, capacity=cap, sched=sched, plan_ahead=plan_ahead)
    r._ensure(n, cap)
    r.splats[:n].copy_(dev(ref["splats"]))
    return r


def plan_fields(p):
    return {k: p[k] for k in ("h", "k", "nA", "order", "counts", "qoff", "qa", "items")}


@pytest.mark.parametrize("cfg", [1, 2])
def test_tile_counts_equal_the_oracle(cfg):
    gsr = _gsr()
    sc, ref = reference(cfg)
    r = rasterizer(gsr, sc, ref)
    r.bin_and_sort(sc.n)
    want = np.diff(ref["ranges"], axis=1)[:, 0]
    assert np.array_equal(host(r.tile_counts), want)
    assert np.array_equal(host(r.ranges), ref["ranges"])


def test_tile_counts_of_a_batch_of_views():
    gsr = _gsr()
    sc = scenegen.random_scene(31, 700, 197, 83, 150.0)
    ref = oracle.frame(sc)
    n = sc.n
    r = gsr.Rasterizer(sc.camera, capacity=max(len(ref["sorted_ids"]), 1) * 2, n_views=2)
    r._ensure(2 * n, r.capacity)
    sp = np.concatenate([ref["splats"], ref["splats"]]).copy()
    sp[n:, 11] = np.array([1], np.int32).view(np.float32)[0]  # view 1's records
    r.splats[:2 * n].copy_(dev(sp))
    r.bin_and_sort(2 * n)
    one = np.diff(ref["ranges"], axis=1)[:, 0]
    assert np.array_equal(host(r.tile_counts), np.concatenate([one, one]))


SCHEDS = {
    "policy": dict(chunk_mode=1),
    "plain": dict(chunk_mode=0),
    "forced": dict(chunk_mode=2, force_k=4, force_h=5),
}


@pytest.mark.parametrize("name", list(SCHEDS))
@pytest.mark.parametrize("cfg", [1, 2])
def test_plan_ahead_equals_the_forward_plan(cfg, name):
    gsr = _gsr()
    sc, ref = reference(cfg)
    out = {}
    for ahead in (True, False):
        r = rasterizer(gsr, sc, ref, sched=gsr.make_sched(**SCHEDS[name]), plan_ahead=ahead)
        r.run_frame(sc.n)
        out[ahead] = (plan_fields(read_plan(r)), host(r.rgb), host(r.T), host(r.last))
    pa, pb = out[True][0], out[False][0]
    for k in pa:
        assert np.array_equal(pa[k], pb[k]), k
    check_queues(read_plan(r), (sc.camera.width + 15) // 16)
    for a, b in zip(out[True][1:], out[False][1:]):
        assert np.array_equal(a, b)


def test_forward_uses_a_plan_built_ahead():
    """A plan built from other counts with the same total orders the tiles by
    those counts; the forward takes it as it is, and the images do not change
    (without chunks, each quarter's blend does not depend on the order)."""
    gsr = _gsr()
    sc, ref = reference(2)
    sched = gsr.make_sched(chunk_mode=0)
    r = rasterizer(gsr, sc, ref, sched=sched, plan_ahead=False)
    r.run_frame(sc.n)
    base = (host(r.rgb), host(r.T), host(r.last))
    counts = np.diff(ref["ranges"], axis=1)[:, 0].astype(np.int32)
    fake = counts[::-1].copy()  # same total, another order
    r.enqueue_bin_sort(sc.n)
    gsr.gs_plan_tiles(dev(fake), r.cam, sched, r.fwd_state, r.status)
    r.render_fwd(sc.n)
    r.check("frame with a plan built ahead")
    plan = read_plan(r)
    T = len(counts)
    want = np.lexsort((np.arange(T), -fake.astype(np.int64)))
    assert np.array_equal(plan["order"], want)
    assert np.array_equal(plan["counts"], fake[want])
    assert not np.array_equal(want, np.lexsort((np.arange(T), -counts.astype(np.int64))))
    for a, b in zip((host(r.rgb), host(r.T), host(r.last)), base):
        assert np.array_equal(a, b)


def test_plan_for_another_pair_total_is_reported():
    gsr = _gsr()
    sc, ref = reference(1)
    r = rasterizer(gsr, sc, ref, plan_ahead=False, cap=4 * len(ref["sorted_ids"]))
    r.enqueue_bin_sort(sc.n)
    counts = np.diff(ref["ranges"], axis=1)[:, 0].astype(np.int32)
    counts[0] += 1
    gsr.gs_plan_tiles(dev(counts), r.cam, r.sched, r.fwd_state, r.status)
    r.rgb.fill_(7.0)
    r.render_fwd(sc.n)
    st, _ = r.frame_status(sc.n)
    assert st == gsr.GS_ERR_WORKSPACE
    assert read_plan(r)["run_f"] == 0
    assert torch.all(r.rgb == 7.0).item()  # the forward did nothing


def test_plan_with_other_knobs_is_rebuilt():
    gsr = _gsr()
    sc, ref = reference(2)
    r = rasterizer(gsr, sc, ref, sched=gsr.make_sched(chunk_mode=0), plan_ahead=False)
    r.enqueue_bin_sort(sc.n)
    counts = np.diff(ref["ranges"], axis=1)[:, 0].astype(np.int32)
    gsr.gs_plan_tiles(dev(counts), r.cam, gsr.make_sched(chunk_mode=0), r.fwd_state, r.status)
    r.sched = gsr.make_sched(chunk_mode=2, force_k=8, force_h=3)
    r.render_fwd(sc.n)
    r.check("frame whose plan was built with other knobs")
    plan = read_plan(r)
    assert (plan["h"], plan["k"]) == (3, 8)


def test_plan_over_the_state_capacity_is_reported():
    gsr = _gsr()
    sc, ref = reference(1)
    r = rasterizer(gsr, sc, ref, plan_ahead=False)
    r.enqueue_bin_sort(sc.n)
    counts = np.diff(ref["ranges"], axis=1)[:, 0].astype(np.int32)
    counts[0] += 1 << 22  # far beyond the capacity the state was sized for
    gsr.gs_plan_tiles(dev(counts), r.cam, r.sched, r.fwd_state, r.status)
    r.render_fwd(sc.n)
    st, _ = r.frame_status(sc.n)
    assert st == gsr.GS_ERR_WORKSPACE


# ---------------------------------------------------------------- planned: checked in the launch

def _planned_forward(gsr, r, n, sched):
    gsr.gs_render_fwd(n, r.splats, r.sorted_ids, r.ranges, r.cam, gsr.planned_sched(sched), r.rgb,
                      r.T, r.last, r.fwd_state, None, None, r.status)


@pytest.mark.parametrize("cfg", [1, 2])
def test_planned_forward_equals_the_handed_over_one(cfg):
    """With sched.planned the forward checks the plan built ahead inside its own
    launch (no hand-over launch): the same plan, the same images bit for bit."""
    gsr = _gsr()
    sc, ref = reference(cfg)
    out = {}
    for planned in (False, True):
        r = rasterizer(gsr, sc, ref, plan_ahead=False)
        r.enqueue_bin_sort(sc.n)
        counts = np.diff(ref["ranges"], axis=1)[:, 0].astype(np.int32)
        gsr.gs_plan_tiles(dev(counts), r.cam, r.sched, r.fwd_state, r.status)
        if planned:
            _planned_forward(gsr, r, sc.n, r.sched)
        else:
            r.render_fwd(sc.n)
        r.check(f"planned={planned}")
        g = host(r.render_bwd(sc.n, dev(sc.dL_drgb))).copy()
        r.check(f"planned={planned} backward")
        out[planned] = (plan_fields(read_plan(r)), host(r.rgb), host(r.T), host(r.last), g)
    for k in out[True][0]:
        assert np.array_equal(np.asarray(out[True][0][k]), np.asarray(out[False][0][k])), k
    for a, b in zip(out[True][1:4], out[False][1:4]):
        assert np.array_equal(a, b)
    rel = np.linalg.norm(out[True][4] - out[False][4], axis=0) / np.linalg.norm(out[False][4], axis=0)
    assert np.all(rel <= 1e-5)


def test_planned_forward_without_a_plan_is_reported():
    """sched.planned on a state that holds no plan built ahead: GS_ERR_WORKSPACE,
    the forward renders nothing and the backward adds nothing."""
    gsr = _gsr()
    sc, ref = reference(1)
    r = rasterizer(gsr, sc, ref, plan_ahead=False)
    r.enqueue_bin_sort(sc.n)
    r.clear_state()
    r.rgb.fill_(7.0)
    _planned_forward(gsr, r, sc.n, r.sched)
    g = r.render_bwd(sc.n, dev(sc.dL_drgb))
    st, _ = r.frame_status(sc.n)
    assert st == gsr.GS_ERR_WORKSPACE
    assert torch.all(r.rgb == 7.0).item() and np.all(host(g) == 0)


def test_planned_forward_with_other_knobs_is_reported():
    gsr = _gsr()
    sc, ref = reference(2)
    r = rasterizer(gsr, sc, ref, sched=gsr.make_sched(chunk_mode=0), plan_ahead=False)
    r.enqueue_bin_sort(sc.n)
    counts = np.diff(ref["ranges"], axis=1)[:, 0].astype(np.int32)
    gsr.gs_plan_tiles(dev(counts), r.cam, gsr.make_sched(chunk_mode=0), r.fwd_state, r.status)
    _planned_forward(gsr, r, sc.n, gsr.make_sched(chunk_mode=2, force_k=8, force_h=3))
    st, _ = r.frame_status(sc.n)
    assert st == gsr.GS_ERR_WORKSPACE


# ---------------------------------------------------------------- the plan built inside the sort

@pytest.mark.parametrize("name", list(SCHEDS))
@pytest.mark.parametrize("size", [(600, 400), (1601, 1399), (256, 256)])
def test_plan_built_in_the_sort_equals_the_forward_plan(size, name):
    """gs_sort_keys_plan builds the schedule in a spare workgroup of its 5-bit
    tile pass (600x400: 950 tiles), or after the sort when the frame has no such
    pass (1601x1399: 8888 tiles; 256x256: 256 tiles); a planned forward uses it.
    The plan equals the one the forward builds itself, field for field, and the
    images are the same bit for bit."""
    gsr = _gsr()
    W, H = size
    sc = scenegen.random_scene(41, 20000, W, H, 0.9 * W)
    ref = oracle.frame(sc)
    out = {}
    for ahead in (True, False):
        r = rasterizer(gsr, sc, ref, sched=gsr.make_sched(**SCHEDS[name]), plan_ahead=ahead)
        r.run_frame(sc.n)
        out[ahead] = (plan_fields(read_plan(r)), host(r.rgb), host(r.T), host(r.last))
    pa, pb = out[True][0], out[False][0]
    for k in pa:
        assert np.array_equal(pa[k], pb[k]), k
    check_queues(read_plan(r), (W + 15) // 16)
    for a, b in zip(out[True][1:], out[False][1:]):
        assert np.array_equal(a, b)
