"""gs_render_fwd_zero (the forward clearing an array in its workers' idle time)
with gs_render_bwd_accumulate adding into it, through the C ABI.

  equal       on a frame whose backward items the forward files in bins
              (garden, urban with its chunks) and on one whose preparation
              orders them (small): the gradients match the oracle, and the
              plain overwriting backward within the order of the float sums
  again       the backward run a second time on the same state adds the same
              gradients again (its queue heads are reset for a re-run)
  cleared     every element of the array is zero after the forward, a ragged
              count included, and nothing past it is written; a frame that
              failed earlier only clears
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from test_gpu_parity import (_gsr, check_backward, check_bwd_queue, dev, host, read_bwd_queue,
                             read_plan, reference)

pytestmark = pytest.mark.gpu


def _rel(a, b):
    a, b = a.astype(np.float64), b.astype(np.float64)
    return np.linalg.norm(a - b, axis=0) / np.maximum(np.linalg.norm(b, axis=0), 1e-30)


def _frame(gsr, sc, ref):
    """The oracle's splats, binned and sorted on the GPU, forward state cleared."""
    n = sc.n
    r = gsr.Rasterizer(sc.camera, capacity=max(len(ref["sorted_ids"]), 1))
    r._ensure(n, r.capacity)
    r.splats[:n].copy_(dev(ref["splats"]))
    r.bin_and_sort(n)
    r.clear_state()
    return r, n, dev(sc.dL_drgb)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_cleared_forward_and_accumulating_backward(cfg):
    gsr = _gsr()
    sc, ref = reference(cfg)
    r, n, dL = _frame(gsr, sc, ref)
    print(f"config {cfg}: forward with clearing", flush=True)
    r.grads.fill_(float("nan"))
    r.render_fwd(n, clear_grads=True)
    assert np.all(host(r.grads)[:n] == 0)
    g1 = host(r.render_bwd(n, dL, accumulate=True)).copy()
    r.check("cleared frame")
    groups, sub_last, qcut, bins = read_bwd_queue(r)
    few = cfg == 2
    assert (bins is None) == few
    items = np.concatenate(groups)
    plan = read_plan(r)
    print(f"config {cfg}: backward items {len(items)}, chunk quarters {int(np.sum((items >> 30) & 3 == 2))}"
          f" of {4 * plan['h'] * plan['k']}, quarter items {int(np.sum((items >> 30) & 3 == 3))}",
          flush=True)
    assert int(np.sum(((items >> 30) & 3) == 2)) == 4 * plan["h"] * plan["k"]
    check_bwd_queue(groups, sub_last, qcut, bins, ref["ranges"], few)
    out = dict(grads=g1)
    check_backward(ref, out)
    # again on the same state: the same gradients added a second time
    g2 = host(r.render_bwd(n, dL, accumulate=True)).copy()
    assert np.all(_rel(g2, 2.0 * g1.astype(np.float64)) <= 1e-5)
    # the plain overwriting backward on the same state
    plain = host(r.render_bwd(n, dL)).copy()
    assert np.all(_rel(g1, plain) <= 1e-5)
    r.check("cleared frame, backward again")


def test_clear_of_a_ragged_count_writes_nothing_past_it():
    gsr = _gsr()
    sc, ref = reference(1)
    r, n, dL = _frame(gsr, sc, ref)
    buf = torch.full((3 * 4096 + 77 + 64,), 7.0, dtype=torch.float32, device="cuda")
    cnt = 3 * 4096 + 77
    gsr.gs_render_fwd_zero(n, r.splats, r.sorted_ids, r.ranges, r.cam, r.sched, r.rgb, r.T,
                           r.last, r.fwd_state, None, None, r.status, buf[:cnt])
    b = host(buf)
    assert np.all(b[:cnt] == 0) and np.all(b[cnt:] == 7.0)
    r.check("ragged clear")


def test_a_failed_frame_only_clears():
    gsr = _gsr()
    sc, ref = reference(2)
    r, n, dL = _frame(gsr, sc, ref)
    r.status.fill_(gsr.GS_ERR_CAPACITY)
    r.rgb.fill_(3.0)
    r.grads.fill_(5.0)
    gsr.gs_render_fwd_zero(n, r.splats, r.sorted_ids, r.ranges, r.cam, r.sched, r.rgb, r.T,
                           r.last, r.fwd_state, None, None, r.status, r.grads[:n])
    assert np.all(host(r.grads)[:n] == 0) and np.all(host(r.grads)[n:] == 5.0)
    assert np.all(host(r.rgb) == 3.0)
    gsr.gs_render_bwd_accumulate(n, r.splats, r.sorted_ids, r.ranges, r.cam, 1, r.T, r.last,
                                 r.fwd_state, dL, r.grads, r.status)
    assert np.all(host(r.grads)[:n] == 0)
    assert int(host(r.status)[0]) == gsr.GS_ERR_CAPACITY


@pytest.mark.parametrize("cfg", [3, 5, 2])
def test_the_benchmarked_chain_matches_the_oracle(cfg):
    """Rasterizer.run_frame with dL/dC, the chain bench.py times: bin, the sort
    with the schedule built inside it (garden and urban, from the second frame
    on; small builds it beside the sort), the planned forward that clears the
    gradient rows, the accumulating backward. Image, transmittance, last entry
    and gradients against the oracle, on the oracle's splat records, for two
    frames in a row (the counting forward: the same images bit for bit)."""
    from test_gpu_parity import check_forward
    gsr = _gsr()
    sc, ref = reference(cfg)
    n = sc.n
    r = gsr.Rasterizer(sc.camera, capacity=max(len(ref["sorted_ids"]), 1))
    r._ensure(n, r.capacity)
    r.splats[:n].copy_(dev(ref["splats"]))
    dL = dev(sc.dL_drgb)
    for frame in range(2):
        r.grads.fill_(float("nan"))
        I = r.run_frame(n, dL, stats=True)
        assert I == len(ref["sorted_ids"])
        in_sort = gsr.plan_in_sort(r.tiles, I) and frame == 1
        print(f"config {cfg} frame {frame}: schedule built "
              f"{'inside' if in_sort else 'beside'} the sort", flush=True)
        out = dict(rgb=host(r.rgb), T=host(r.T), last=host(r.last), grads=host(r.grads)[:n].copy(),
                   pixel_hits=host(r.pixel_hits), stats=host(r.stats))
        check_forward(ref, out)
        check_backward(ref, out)
