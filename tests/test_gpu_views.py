"""Batches of views (the *_views calls) against one oracle frame per view.

A batch of V cameras of one size is binned, sorted and rendered as one image:
view v's records, tiles and pixel rows follow those of view v - 1, and one
persistent forward and one backward launch serve every view's tiles. Each
view's results must equal the single-view oracle's for that view, to the
single-view bars: records within the projection tolerance, pairs, sorted keys,
ids and ranges bit-exact, rgb and T within 1e-5, gradients within 1e-3
relative L2 per column; the projection backward sums the views.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import scenegen
from test_gpu_parity import (_gsr, check_backward, check_binning, check_forward, check_projection,
                             check_sort, dev, host)
from test_gpu_project_bwd import NAMES

pytestmark = pytest.mark.gpu


def _rot(rng, s):
    ang = rng.normal(0, s, 3)
    q = np.array([1.0, *ang])
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                     [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                     [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def _views(sc, V, seed):
    """V cameras of sc.camera's size: the scene's own and V - 1 moved ones."""
    rng = np.random.default_rng(seed)
    c0 = sc.camera
    cams = [c0]
    for _ in range(V - 1):
        M = np.asarray(c0.world_to_cam, np.float64).reshape(3, 4)
        R = _rot(rng, 0.08) @ M[:, :3]
        t = M[:, 3] + rng.normal(0, 0.1, 3)
        cams.append(scenegen.pinhole(c0.width, c0.height, float(c0.fx),
                                     np.concatenate([R, t[:, None]], 1)))
    dL = [rng.standard_normal((3, c0.height, c0.width)).astype(np.float32) for _ in range(V)]
    return cams, dL


def _run(gsr, sc, cams, ref, dL, sched=None, background=None, dT=None):
    V = len(cams)
    n_rec = sc.n * V
    npairs = len(ref["sorted_ids"])
    r = gsr.Rasterizer(cams[0], capacity=max(npairs, 1), sched=sched, n_views=V)
    r._ensure(n_rec, r.capacity)
    r.splats[:n_rec].copy_(dev(ref["splats"]))
    I = r.bin_and_sort(n_rec, want_keys=True, want_emission=True)
    out = dict(I=I, offsets=host(r.offsets), keys=host(r.keys)[:I].view(np.uint64),
               ids=host(r.ids)[:I], sorted_keys=host(r.sorted_keys)[:I].view(np.uint64),
               sorted_ids=host(r.sorted_ids)[:I], ranges=host(r.ranges))
    r.render_fwd(n_rec, stats=True, background=background)
    dL_all = dev(np.concatenate(dL, axis=1))
    dT_all = None if dT is None else dev(np.concatenate(dT))
    grads = r.render_bwd(n_rec, dL_all, background=background, dL_dT=dT_all)
    r.check("views frame")
    out.update(rgb=host(r.rgb), T=host(r.T), last=host(r.last), grads=host(grads),
               stats=host(r.stats), pixel_hits=host(r.pixel_hits))
    return out


@pytest.mark.parametrize("V", [2, 3])
def test_views_match_one_oracle_frame_per_view(V):
    gsr = _gsr()
    sc = scenegen.make_config(2)
    cams, dL = _views(sc, V, 300 + V)
    ref = oracle.frame_views(sc, cams, dL)
    # the batched projection against the oracle, view by view
    r = gsr.Rasterizer(cams[0], capacity=16, n_views=V)
    sp = host(r.project_views(cams, dev(sc.means), dev(sc.log_scales), dev(sc.quats),
                              dev(sc.opacities), dev(sc.sh), sc.sh_degree)).copy()
    for v in range(V):
        rows = slice(v * sc.n, (v + 1) * sc.n)
        check_projection(sc, ref["splats"][rows], sp[rows])
        assert np.all(sp[rows, 11].view(np.int32) == v)
    del r
    out = _run(gsr, sc, cams, ref, dL)
    check_binning(ref, out)
    check_sort(ref, out)
    check_forward(ref, out)
    check_backward(ref, out)


def test_views_ragged_size_background_and_chunks():
    """A size that is not a multiple of 16 (partial last tile row in every view),
    a background, dL/dT_final and forced depth chunks."""
    gsr = _gsr()
    sc = scenegen.random_scene(106, 3000, 83, 45, 75.0, degree=1, log_scale=(-2.0, 0.6),
                               opacity=(1.0, 2.0))
    cams, dL = _views(sc, 4, 310)
    rng = np.random.default_rng(311)
    bg = rng.uniform(-0.5, 1.0, 3).astype(np.float32)
    dT = [rng.standard_normal((45, 83)).astype(np.float32) for _ in range(4)]
    ref = oracle.frame_views(sc, cams, dL, bg=bg, dL_dTs=dT)
    sched = gsr.make_sched(chunk_mode=2, force_k=4, force_h=20)
    out = _run(gsr, sc, cams, ref, dL, sched=sched, background=bg, dT=dT)
    check_binning(ref, out)
    check_sort(ref, out)
    check_forward(ref, out)
    check_backward(ref, out)


def test_one_view_batch_equals_plain_calls():
    gsr = _gsr()
    sc = scenegen.make_config(2)
    ref = oracle.frame(sc)
    n = sc.n
    npairs = len(ref["sorted_ids"])
    outs = []
    for views in (False, True):
        r = gsr.Rasterizer(sc.camera, capacity=npairs)
        r._ensure(n, npairs)
        r.splats[:n].copy_(dev(ref["splats"]))
        if views:
            gsr.gs_bin_tiles_views(n, r.splats, r.cam, 1, r.capacity, r.offsets, None, None,
                                   r.status, r.workspace)
            gsr.gs_sort_keys_views(n, r.splats, r.offsets, r.capacity, r.cam, 1, None,
                                   r.sorted_ids, r.ranges, r.status, r.workspace)
            gsr.gs_render_fwd_views(n, r.splats, r.sorted_ids, r.ranges, r.cam, 1, r.sched,
                                    r.rgb, r.T, r.last, r.fwd_state, None, None, r.status)
            r.check("one-view batch")
        else:
            r.bin_and_sort(n)
            r.render_fwd(n)
        outs.append((host(r.sorted_ids)[:npairs].copy(), host(r.rgb).copy(), host(r.T).copy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_project_bwd_views_sums_the_views():
    gsr = _gsr()
    sc = scenegen.make_config(2)
    cams, _ = _views(sc, 3, 320)
    rng = np.random.default_rng(321)
    g = rng.normal(0, 1, (3 * sc.n, 9)).astype(np.float32)
    g[rng.random(3 * sc.n) < 0.3] = 0.0
    r = gsr.Rasterizer(cams[0], capacity=16, n_views=3)
    d = [dev(a) for a in (sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh)]
    sp = host(r.project_views(cams, *d, sc.sh_degree)).copy()
    out = {k: host(v) for k, v in r.project_bwd_views(cams, *d, sc.sh_degree,
                                                      dL_dsplat=dev(g)).items()}
    ref = {k: 0.0 for k in NAMES}
    vis_gpu = np.zeros(sc.n, bool)
    vis_ref = np.zeros(sc.n, bool)
    for v, cam in enumerate(cams):
        rows = slice(v * sc.n, (v + 1) * sc.n)
        rv = oracle.project_bwd(sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh,
                                sc.sh_degree, cam, g[rows])
        for k in NAMES:
            ref[k] = ref[k] + rv[k]
        rs = oracle.project(sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh, sc.sh_degree,
                            cam)
        vis_ref |= rs[:, 9] > 0
        vis_gpu |= sp[rows, 9] > 0
    # knife-edge culls (fp32 against fp64) may differ: compare where both agree in every view
    same = np.ones(sc.n, bool)
    for v, cam in enumerate(cams):
        rows = slice(v * sc.n, (v + 1) * sc.n)
        rs = oracle.project(sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh, sc.sh_degree,
                            cam)
        same &= (rs[:, 9] > 0) == (sp[rows, 9] > 0)
    assert (~same).sum() <= 6
    for k in NAMES:
        a = out[k].reshape(sc.n, -1)[same].astype(np.float64)
        b = np.asarray(ref[k]).reshape(sc.n, -1)[same]
        err = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)
        assert err <= 1e-3, (k, err)
        assert np.all(out[k].reshape(sc.n, -1)[~vis_gpu] == 0), k


def test_views_reject_bad_batches():
    gsr = _gsr()
    sc = scenegen.make_config(1)
    cams, _ = _views(sc, 2, 330)
    other = scenegen.pinhole(sc.camera.width + 16, sc.camera.height, float(sc.camera.fx))
    r = gsr.Rasterizer(cams[0], capacity=16, n_views=2)
    d = [dev(a) for a in (sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh)]
    with pytest.raises(gsr.GsError):
        r.project_views([cams[0], other], *d, sc.sh_degree)
    assert gsr.fwd_state_size_views(64, 64, 0, 100) == 0
    assert gsr.fwd_state_size_views(64, 64, 17, 100) == 0
    assert gsr.fwd_state_size_views(64, 64, 2, -1) == 0
    assert gsr.workspace_size_views(10, 64, 64, 17, 100) == 0
