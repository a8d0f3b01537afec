"""gs_render_bwd_accumulate: the backward adding into a gradient array the
caller initialises (the plain calls overwrite theirs), through the C ABI.

  zeroed      on a zeroed array it gives gs_render_bwd's gradients (the sums
              meet in a different order: relative L2 per column within 1e-5)
  on top      on an array holding B it gives B + those gradients
  failed      a frame whose status is not GS_OK adds nothing (bit for bit)
  views       n_views = 2 against gs_render_bwd_views
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import scenegen
from test_gpu_parity import _gsr, dev, host, reference

pytestmark = pytest.mark.gpu


def _rel(a, b):
    a, b = a.astype(np.float64), b.astype(np.float64)
    return np.linalg.norm(a - b, axis=0) / np.maximum(np.linalg.norm(b, axis=0), 1e-30)


def _frame(gsr, sc, ref, n_views=1):
    n = sc.n * n_views
    r = gsr.Rasterizer(sc.camera, capacity=max(len(ref["sorted_ids"]), 1) * n_views,
                       n_views=n_views, plan_ahead=False)
    r._ensure(n, r.capacity)
    sp = np.concatenate([ref["splats"]] * n_views).copy()
    for v in range(n_views):
        sp[v * sc.n:(v + 1) * sc.n, 11] = np.array([v], np.int32).view(np.float32)[0]
    r.splats[:n].copy_(dev(sp))
    r.bin_and_sort(n)
    r.render_fwd(n)
    dL = dev(np.concatenate([sc.dL_drgb] * n_views, axis=1))
    return r, n, dL


def _accumulate(gsr, r, n, dL, out):
    gsr.gs_render_bwd_accumulate(n, r.splats, r.sorted_ids, r.ranges, r.cam, r.V, r.T, r.last,
                                 r.fwd_state, dL, out, r.status)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [1, 2])
def test_accumulate_on_zeros_equals_the_plain_backward(cfg):
    gsr = _gsr()
    sc, ref = reference(cfg)
    r, n, dL = _frame(gsr, sc, ref)
    plain = host(r.render_bwd(n, dL)).copy()
    acc = torch.zeros_like(r.grads)
    _accumulate(gsr, r, n, dL, acc)
    assert np.all(_rel(host(acc)[:n], plain) <= 1e-5)
    assert np.all(_rel(plain, ref["grads"]) <= 1e-3)


def test_accumulate_adds_to_what_the_array_holds():
    gsr = _gsr()
    sc, ref = reference(2)
    r, n, dL = _frame(gsr, sc, ref)
    plain = host(r.render_bwd(n, dL)).astype(np.float64)
    rng = np.random.default_rng(5)
    base = (rng.standard_normal(r.grads.shape) * np.abs(plain).max()).astype(np.float32)
    acc = dev(base)
    _accumulate(gsr, r, n, dL, acc)
    got = host(acc)[:n].astype(np.float64) - base[:n]
    scale = np.abs(base[:n]).max() + np.abs(plain).max()
    assert np.abs(got - plain).max() <= 1e-5 * scale


def test_accumulate_on_a_failed_frame_adds_nothing():
    gsr = _gsr()
    sc, ref = reference(2)
    r, n, dL = _frame(gsr, sc, ref)
    base = np.random.default_rng(6).standard_normal(r.grads.shape).astype(np.float32)
    acc = dev(base)
    r.status.fill_(gsr.GS_ERR_CAPACITY)
    _accumulate(gsr, r, n, dL, acc)
    assert np.array_equal(host(acc), base)


def test_accumulate_for_a_batch_of_views():
    gsr = _gsr()
    sc = scenegen.random_scene(33, 900, 141, 77, 120.0)
    ref = oracle.frame(sc, fwd=False)
    r, n, dL = _frame(gsr, sc, ref, n_views=2)
    plain = host(r.render_bwd(n, dL)).copy()
    acc = torch.zeros_like(r.grads)
    _accumulate(gsr, r, n, dL, acc)
    assert np.all(_rel(host(acc)[:n], plain) <= 1e-5)
    # each view's rows carry that view's gradients: the two halves agree
    assert np.all(_rel(plain[sc.n:], plain[:sc.n]) <= 1e-5)
