"""Edge cases of the raster stages, on crafted splat records, against the oracle.

Each case builds records directly (the projection is covered elsewhere) and
runs the GPU stages on them with the single-view bars: pairs, sorted keys, ids
and ranges bit-exact; rgb and T within 1e-5; gradients within 1e-3 relative L2
per column. Cases: opacities at the 1/255 cutoff and in the 0.99 clamp, depth
ties (order by Gaussian id), a splat covering the whole screen under many
small ones, needle-thin splats, every splat in one tile (which the policy of
"Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
section 4.4 chunks), and repeated runs (the forward and the sort are
deterministic; the backward's float atomics only reorder additions).
"""
import math
import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import scenegen
from test_gpu_parity import (_gsr, check_backward, check_binning, check_forward, check_sort,
                             run_stages)

pytestmark = pytest.mark.gpu


def _records(rng, n, W, H, sig=(1.0, 6.0), o=(0.05, 0.95), aniso=1.0):
    s = np.zeros((n, 12), np.float32)
    s[:, 0] = rng.uniform(-4, W + 4, n)
    s[:, 1] = rng.uniform(-4, H + 4, n)
    sx = rng.uniform(*sig, n)
    sy = sx / aniso
    th = rng.uniform(0, np.pi, n)
    c, sn = np.cos(th), np.sin(th)
    sxx = c * c * sx ** 2 + sn * sn * sy ** 2
    syy = sn * sn * sx ** 2 + c * c * sy ** 2
    sxy = c * sn * (sx ** 2 - sy ** 2)
    det = sxx * syy - sxy ** 2
    s[:, 2], s[:, 3], s[:, 4] = syy / det, -sxy / det, sxx / det
    s[:, 5] = rng.uniform(*o, n)
    s[:, 6:9] = rng.uniform(0, 1, (n, 3))
    s[:, 9] = (2 * np.log(255 * s[:, 5].astype(np.float64))).astype(np.float32)
    s[:, 10] = rng.uniform(1, 5, n)
    return s


def _frame(s, W, H, seed):
    """The oracle's frame on given records; a scene stand-in for run_stages."""
    cam = scenegen.pinhole(W, H, float(W))
    dL = np.random.default_rng(seed).standard_normal((3, H, W)).astype(np.float32)
    off, keys, ids = oracle.bin_tiles(s, W, H)
    sk, si = oracle.sort_pairs(keys, ids)
    rng_ = oracle.tile_ranges(sk, cam.num_tiles)
    f = oracle.render_fwd(s, si, rng_, W, H)
    g = oracle.render_bwd(s, si, rng_, W, H, f["last"], dL)
    ref = dict(splats=s, offsets=off, keys=keys, ids=ids, sorted_keys=sk, sorted_ids=si,
               ranges=rng_, fwd=f, grads=g)
    sc = types.SimpleNamespace(camera=cam, n=len(s), dL_drgb=dL)
    return sc, ref


def _check_all(gsr, sc, ref, sched=None):
    out = run_stages(gsr, sc, ref, sched=sched)
    check_binning(ref, out)
    check_sort(ref, out)
    check_forward(ref, out)
    check_backward(ref, out)
    return out


def test_opacity_at_the_cutoff_and_in_the_clamp():
    gsr = _gsr()
    rng = np.random.default_rng(400)
    W, H = 97, 61
    s = _records(rng, 1500, W, H)
    k = len(s) // 3
    s[:k, 5] = (1 / 255) * (1 + rng.uniform(-2e-3, 2e-3, k))      # tau near 0, either side
    s[k:2 * k, 5] = rng.uniform(0.985, 1.0, k)                      # alpha clamped at 0.99
    s[:, 9] = (2 * np.log(255 * s[:, 5].astype(np.float64))).astype(np.float32)
    assert (s[:k, 9] <= 0).any() and (s[:k, 9] > 0).any()
    _check_all(gsr, *_frame(s, W, H, 401))


def test_depth_ties_order_by_gaussian_id():
    gsr = _gsr()
    rng = np.random.default_rng(410)
    W, H = 64, 48
    s = _records(rng, 1200, W, H)
    s[:, 10] = rng.choice(np.array([1.5, 2.0, 2.5], np.float32), len(s))   # three depths only
    sc, ref = _frame(s, W, H, 411)
    out = _check_all(gsr, sc, ref)
    # inside every tile, equal depths appear in increasing id order
    ids, keys = out["sorted_ids"], out["sorted_keys"]
    same = (keys[1:] == keys[:-1])
    assert same.any() and np.all(ids[1:][same] > ids[:-1][same])


def test_screen_covering_splat_under_small_ones():
    gsr = _gsr()
    rng = np.random.default_rng(420)
    W, H = 150, 90
    s = _records(rng, 2000, W, H, sig=(0.5, 3.0))
    big = np.zeros(12, np.float32)
    big[:6] = [W / 2, H / 2, 1 / 200.0 ** 2, 0, 1 / 200.0 ** 2, 0.8]
    big[6:9] = [0.2, 0.4, 0.6]
    big[9] = 2 * math.log(255 * 0.8)
    big[10] = 10.0                                   # behind every small splat
    s = np.concatenate([s, big[None]])
    sc, ref = _frame(s, W, H, 421)
    out = _check_all(gsr, sc, ref)
    assert int(out["offsets"][-1] - out["offsets"][-2]) == sc.camera.num_tiles


def test_needle_thin_splats():
    gsr = _gsr()
    rng = np.random.default_rng(430)
    W, H = 120, 80
    s = _records(rng, 1500, W, H, sig=(3.0, 30.0), aniso=80.0)
    _check_all(gsr, *_frame(s, W, H, 431))


def test_every_splat_in_one_tile_is_chunked():
    gsr = _gsr()
    rng = np.random.default_rng(440)
    W, H = 128, 96
    n = 6000
    s = _records(rng, n, W, H, sig=(0.3, 1.2), o=(0.01, 0.05))
    s[:, 0] = rng.uniform(40.5, 47.5, n)            # all inside tile (2, 3)
    s[:, 1] = rng.uniform(56.5, 63.5, n)
    sc, ref = _frame(s, W, H, 441)
    counts = ref["ranges"][:, 1] - ref["ranges"][:, 0]
    assert counts.max() >= 5000
    out = _check_all(gsr, sc, ref, sched=gsr.make_sched(chunk_mode=1))
    assert int(out["stats"][3]) >= 1                 # the policy split the outlier tile


def test_repeated_runs_are_deterministic():
    gsr = _gsr()
    sc = scenegen.make_config(2)
    ref = oracle.frame(sc)
    a = run_stages(gsr, sc, ref)
    b = run_stages(gsr, sc, ref)
    for k in ("offsets", "keys", "ids", "sorted_keys", "sorted_ids", "ranges", "last"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("rgb", "T"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    ga, gb = a["grads"].astype(np.float64), b["grads"].astype(np.float64)
    rel = np.linalg.norm(ga - gb, axis=0) / np.maximum(np.linalg.norm(ga, axis=0), 1e-30)
    assert np.all(rel <= 1e-6), rel
