"""Pins of the oracle's forward blend and analytic backward.

Forward: "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
section 2.1 Eq. 2-3 (alpha = o exp(-q/2); C = sum c_i alpha_i T_i; stop once T
falls below 1e-4). Backward: "What the 3DGS Literature Left on the Table",
Step 1 (a) (9 screen-space gradients: centre x/y, conic a/b/c, opacity, RGB),
Step 1 (e) (scalar accumulator accum = c_behind . dL/dC), Step 6.3 (the
per-splat gradient alpha T (c . dL/dC - accum)).
"""
import math

import numpy as np
import pytest

import oracle
import scenegen


def _frame_from_splats(s, W, H):
    off, keys, ids = oracle.bin_tiles(s, W, H)
    sk, si = oracle.sort_pairs(keys, ids)
    r = oracle.tile_ranges(sk, ((W + 15) // 16) * ((H + 15) // 16))
    return si, r


def _splat(mx, my, sigma, o, rgb, depth, tau=None):
    s = np.zeros(12, np.float32)
    s[:6] = [mx, my, 1 / sigma ** 2, 0, 1 / sigma ** 2, o]
    s[6:9] = rgb
    s[9] = 2 * math.log(255 * o) if tau is None else tau
    s[10] = depth
    return s


def _alpha_closed(s, px, py):
    """alpha at pixel centres for an isotropic splat (fp64 closed form)."""
    r2 = (px + 0.5 - s[0]) ** 2 + (py + 0.5 - s[1]) ** 2
    sig2 = 1.0 / float(s[2])
    a = np.minimum(0.99, float(s[5]) * np.exp(-r2 / (2 * sig2)))
    return np.where(r2 / sig2 <= float(s[9]), a, 0.0)


def test_single_isotropic_closed_form():
    W, H = 45, 37
    s = _splat(20.3, 17.8, 4.0, 0.8, [0.5, -0.25, 1.0], 3.0)[None]
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    py, px = np.mgrid[0:H, 0:W]
    al = _alpha_closed(s[0], px, py)
    for ch in range(3):
        np.testing.assert_allclose(f["rgb"][ch], s[0, 6 + ch] * al, atol=2e-7)
    np.testing.assert_allclose(f["T"], 1 - al, atol=2e-7)
    assert f["hits"] == int((al > 0).sum())


def test_two_splats_closed_form_and_order():
    W, H = 40, 40
    s1 = _splat(18.0, 20.0, 5.0, 0.7, [1.0, 0.0, 0.0], 2.0)
    s2 = _splat(22.0, 19.0, 6.0, 0.6, [0.0, 1.0, 0.5], 1.0)   # nearer: blended first
    s = np.stack([s1, s2])
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    py, px = np.mgrid[0:H, 0:W]
    a1, a2 = _alpha_closed(s1, px, py), _alpha_closed(s2, px, py)
    for ch in range(3):
        ref = s2[6 + ch] * a2 + s1[6 + ch] * a1 * (1 - a2)
        np.testing.assert_allclose(f["rgb"][ch], ref, atol=3e-7)
    np.testing.assert_allclose(f["T"], (1 - a1) * (1 - a2), atol=3e-7)


def test_white_splats_give_one_minus_T():
    sc = scenegen.random_scene(21, 300, 50, 41, 50.0, log_scale=(-2.5, 0.4))
    s = oracle.project_scene(sc)
    s[:, 6:9] = 1.0
    si, r = _frame_from_splats(s, 50, 41)
    f = oracle.render_fwd(s, si, r, 50, 41)
    for ch in range(3):
        np.testing.assert_allclose(f["rgb"][ch], 1.0 - f["T"], atol=2e-6)


def test_stop_rule_includes_the_crossing_splat():
    """Opaque splats centred on a pixel centre: alpha = 0.99 exactly there;
    T = (1 - 0.99f)^2 < 1e-4 after two, so the third is not blended."""
    W, H = 16, 16
    s = np.stack([_splat(8.5, 8.5, 2.0, 0.99, [1, 0, 0], 1.0),
                  _splat(8.5, 8.5, 2.0, 0.99, [0, 1, 0], 2.0),
                  _splat(8.5, 8.5, 2.0, 0.99, [0, 0, 1], 3.0)])
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    t1 = np.float32(1) - np.float32(0.99)
    assert f["last"][8, 8] == 2
    assert f["T"][8, 8] == np.float32(t1 * t1) < 1e-4
    assert f["rgb"][0, 8, 8] == np.float32(0.99)
    assert f["rgb"][1, 8, 8] == np.float32(np.float32(0.99) * t1)
    assert f["rgb"][2, 8, 8] == 0.0
    # pixels that never stop consumed the whole tile list
    assert f["last"][0, 0] == 3


@pytest.mark.parametrize("seed,W,H,n", [(31, 64, 64, 500), (32, 83, 45, 800), (33, 17, 70, 900)])
def test_tiled_equals_untiled_bitwise(seed, W, H, n):
    """Tiling, binning and sorting change nothing: the untiled walk over every
    visible splat in (depth, id) order gives bit-identical pixels."""
    sc = scenegen.random_scene(seed, n, W, H, 0.9 * W, degree=1, log_scale=(-1.5, 0.5),
                               opacity=(1.0, 2.0))
    s = oracle.project_scene(sc)
    s[::7, 10] = s[3, 10]                          # force exact depth ties
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    rgb_u, T_u, hits_u = oracle.render_fwd_untiled(s, W, H, want_hits=True)
    assert np.array_equal(f["rgb"], rgb_u)
    assert np.array_equal(f["T"], T_u)
    assert np.array_equal(f["pixel_hits"], hits_u)  # the same splats blended, pixel by pixel
    assert f["pixel_hits"].sum() == f["hits"]
    assert (f["T"] < 1e-4).sum() > 0                # the stop rule is exercised


def _f32(x):
    return np.float32(x) if np.isscalar(x) else np.asarray(x, np.float32)


def _fma32(a, b, c):
    """fp32 fused multiply-add: the fp32 product is exact in fp64, and the sum is
    rounded to fp64 then fp32 (a double rounding that differs from a single one
    only at a fp32 midpoint, which these inputs never reach in practice)."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) +
            np.asarray(c, np.float64)).astype(np.float32)


def _hits_numpy(s, si, r, W, H, last):
    """Brute force in numpy, independent of the C code: the canonical fp32 q of
    every (pixel, list entry) of its tile before the pixel's stop, and the hit
    decision q <= tau. Returns the per-pixel hit counts and, per list position,
    the bits of the tile quarters with at least one hit."""
    tx = (W + 15) // 16
    hits = np.zeros((H, W), np.int32)
    pq = np.zeros(len(si), np.uint8)
    for t in range(len(r)):
        a0, a1 = int(r[t, 0]), int(r[t, 1])
        if a1 == a0:
            continue
        x0, y0 = 16 * (t % tx), 16 * (t // tx)
        py, px = np.mgrid[y0:min(y0 + 16, H), x0:min(x0 + 16, W)]
        fx, fy = _f32(px + 0.5), _f32(py + 0.5)
        rec = s[si[a0:a1]]                                   # [m, 12]
        dx = fx[None] - rec[:, 0, None, None]
        dy = fy[None] - rec[:, 1, None, None]
        A, B2, Cc = rec[:, 2, None, None], _f32(2) * rec[:, 3, None, None], rec[:, 4, None, None]
        inner = _fma32(B2 * dx, dy, (A * dx) * dx)
        q = _fma32(Cc * dy, dy, inner)
        pos = np.arange(a1 - a0)[:, None, None]
        hit = (q <= rec[:, 9, None, None]) & (pos < last[py, px][None])
        hits[py, px] = hit.sum(axis=0)
        quad = ((px - x0) >> 3) | (((py - y0) >> 3) << 1)
        for qd in range(4):
            anyq = (hit & (quad == qd)[None]).reshape(len(rec), -1).any(axis=1)
            pq[a0:a1] |= (anyq.astype(np.uint8) << qd)
    return hits, pq


@pytest.mark.parametrize("seed,W,H,n", [(41, 64, 64, 600), (42, 83, 45, 900)])
def test_pixel_hits_and_quarter_contributors_brute_force(seed, W, H, n):
    """The per-pixel hit counts and the per-quarter contributor bits of every
    list position ([3DGS-CUDA] Step 4: which splats blended into which part of
    a tile) equal an independent numpy evaluation of the canonical q."""
    sc = scenegen.random_scene(seed, n, W, H, 0.9 * W, degree=1, log_scale=(-1.5, 0.5),
                               opacity=(1.0, 2.0))
    s = oracle.project_scene(sc)
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    hits, pq = _hits_numpy(s, si, r, W, H, f["last"])
    assert np.array_equal(f["pixel_hits"], hits)
    assert np.array_equal(f["pair_quarters"], pq)
    assert 0 < (pq == 0).sum() < len(pq)          # some positions blend nowhere (occluded)
    assert len(np.unique(pq)) >= 8                 # many quarter combinations occur


def test_backward_is_deterministic_across_thread_counts():
    """The oracle's per-splat sums run in a fixed order: 1, 3 and 8 threads give
    the same bits."""
    sc = scenegen.random_scene(44, 1500, 83, 45, 70.0, degree=1, log_scale=(-1.5, 0.5),
                               opacity=(1.0, 2.0))
    s = oracle.project_scene(sc)
    si, r = _frame_from_splats(s, 83, 45)
    f = oracle.render_fwd(s, si, r, 83, 45)
    outs = []
    before = oracle.num_threads()
    try:
        for nt in (1, 3, 8):
            oracle.set_num_threads(nt)
            outs.append(oracle.render_bwd(s, si, r, 83, 45, f["last"], sc.dL_drgb))
    finally:
        oracle.set_num_threads(before)
    assert np.any(outs[0] != 0)
    for g in outs[1:]:
        assert np.array_equal(g.view(np.uint64), outs[0].view(np.uint64))


def test_transmittance_bounds_and_last():
    sc = scenegen.make_config(1)
    o = oracle.frame(sc, bwd=False)
    f = o["fwd"]
    assert np.all(f["T"] > 0) and np.all(f["T"] <= 1)
    lens = o["ranges"][:, 1] - o["ranges"][:, 0]
    tx = sc.camera.tiles_x
    py, px = np.mgrid[0:sc.camera.height, 0:sc.camera.width]
    tile = (py // 16) * tx + px // 16
    stopped = f["T"] < 1e-4
    assert np.all(f["last"][~stopped] == lens[tile[~stopped]])
    assert np.all(f["last"][stopped] <= lens[tile[stopped]])


# ---------------------------------------------------------------- backward

def _fd_scene(seed, o_range=(0.2, 0.95), n=25, W=37, H=29):
    rng = np.random.default_rng(seed)
    s = np.zeros((n, 12), np.float32)
    s[:, 0] = rng.uniform(2, W - 2, n)
    s[:, 1] = rng.uniform(2, H - 2, n)
    sx, sy = rng.uniform(1.5, 6, n), rng.uniform(1.5, 6, n)
    th = rng.uniform(0, np.pi, n)
    c, sn = np.cos(th), np.sin(th)
    sxx, syy, sxy = c * c * sx ** 2 + sn * sn * sy ** 2, sn * sn * sx ** 2 + c * c * sy ** 2, c * sn * (sx ** 2 - sy ** 2)
    det = sxx * syy - sxy ** 2
    s[:, 2], s[:, 3], s[:, 4] = syy / det, -sxy / det, sxx / det
    s[:, 5] = rng.uniform(*o_range, n)
    s[:, 6:9] = rng.uniform(-1, 1, (n, 3))
    s[:, 9] = 2 * np.log(255 * s[:, 5].astype(np.float64))
    s[:, 10] = rng.uniform(1, 5, n)
    g = rng.standard_normal((3, H, W)).astype(np.float32)
    return s, g, W, H


@pytest.mark.parametrize("seed,o_range,n", [(41, (0.2, 0.95), 25), (42, (0.6, 1.0), 90)])
def test_backward_matches_central_differences(seed, o_range, n):
    s, g, W, H = _fd_scene(seed, o_range, n)
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    assert (f["T"] < 1e-4).sum() > 0 or seed == 41
    grads = oracle.render_bwd(s, si, r, W, H, f["last"], g)
    base = s.astype(np.float64)
    g64 = g.astype(np.float64)
    fd = np.zeros_like(grads)
    for i in range(len(s)):
        for j in range(9):
            h = 1e-6 * max(1.0, abs(base[i, j]))
            vals = []
            for sign in (1, -1):
                v = base.copy()
                v[i, j] += sign * h
                rgb, _ = oracle.render_fwd_values(s, v, si, r, W, H, f["last"])
                vals.append(float((rgb * g64).sum()))
            fd[i, j] = (vals[0] - vals[1]) / (2 * h)
    scale = np.abs(grads).max(axis=0) + 1e-12
    err = np.abs(fd - grads) / scale
    assert err.max() < 1e-6, (err.max(axis=0))
    assert np.all(np.abs(grads).max(axis=0) > 1e-3)     # every parameter receives gradient


def test_backward_linear_in_upstream_gradient():
    s, g1, W, H = _fd_scene(43)
    g2 = np.random.default_rng(44).standard_normal(g1.shape).astype(np.float32)
    # dyadic values so that g1 + 2 g2 is exact in fp32
    g1 = (np.round(g1 * 1024) / 1024).astype(np.float32)
    g2 = (np.round(g2 * 1024) / 1024).astype(np.float32)
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    G1 = oracle.render_bwd(s, si, r, W, H, f["last"], g1)
    G2 = oracle.render_bwd(s, si, r, W, H, f["last"], g2)
    G12 = oracle.render_bwd(s, si, r, W, H, f["last"], (g1.astype(np.float64) + 2 * g2).astype(np.float32))
    np.testing.assert_allclose(G12, G1 + 2 * G2, rtol=1e-6, atol=1e-9)


def test_backward_symmetry_of_centred_isotropic_splat():
    """Isotropic splat on the pixel corner (16,16) with uniform upstream gradient:
    the centre and off-diagonal conic gradients vanish; a and c get equal gradients."""
    W, H = 32, 32
    s = _splat(16.0, 16.0, 3.0, 0.7, [0.3, 0.6, 0.9], 2.0)[None]
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    g = np.ones((3, H, W), np.float32)
    G = oracle.render_bwd(s, si, r, W, H, f["last"], g)[0]
    assert abs(G[0]) < 1e-12 and abs(G[1]) < 1e-12 and abs(G[3]) < 1e-12
    assert G[2] == pytest.approx(G[4], rel=1e-12)
    # one splat: dL/dc = sum_p alpha_p g_p
    py, px = np.mgrid[0:H, 0:W]
    al = _alpha_closed(s[0], px, py)
    assert G[6] == pytest.approx(al.sum(), rel=1e-6)


def test_backward_zero_for_splats_behind_the_stop():
    W, H = 16, 16
    s = np.stack([_splat(8.5, 8.5, 300.0, 1.0, [1, 0, 0], 1.0),
                  _splat(8.5, 8.5, 300.0, 1.0, [0, 1, 0], 2.0),
                  _splat(8.5, 8.5, 300.0, 1.0, [0, 0, 1], 3.0)])
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H)
    assert np.all(f["last"] == 2)
    G = oracle.render_bwd(s, si, r, W, H, f["last"], np.ones((3, H, W), np.float32))
    assert np.all(G[2] == 0)
    # every hit sits in the alpha = 0.99 clamp: only the colour receives gradient
    assert np.all(G[:2, :6] == 0) and np.all(G[:2, 6] != 0)


# ------------------------------------------------ background and dL/dT_final

def test_background_closed_form_single_splat():
    """C = c alpha + (1 - alpha) bg for one splat; T is unchanged by the background."""
    W, H = 45, 37
    s = _splat(20.3, 17.8, 4.0, 0.8, [0.5, -0.25, 1.0], 3.0)[None]
    si, r = _frame_from_splats(s, W, H)
    bg = np.array([0.25, 0.5, -1.0], np.float32)
    f = oracle.render_fwd(s, si, r, W, H, bg=bg)
    f0 = oracle.render_fwd(s, si, r, W, H)
    py, px = np.mgrid[0:H, 0:W]
    al = _alpha_closed(s[0], px, py)
    for ch in range(3):
        np.testing.assert_allclose(f["rgb"][ch], s[0, 6 + ch] * al + (1 - al) * bg[ch], atol=3e-7)
    assert np.array_equal(f["T"], f0["T"]) and np.array_equal(f["last"], f0["last"])


def test_white_splats_on_white_background_give_one():
    sc = scenegen.random_scene(21, 300, 50, 41, 50.0, log_scale=(-2.5, 0.4))
    s = oracle.project_scene(sc)
    s[:, 6:9] = 1.0
    si, r = _frame_from_splats(s, 50, 41)
    f = oracle.render_fwd(s, si, r, 50, 41, bg=[1.0, 1.0, 1.0])
    np.testing.assert_allclose(f["rgb"], 1.0, atol=2e-6)


@pytest.mark.parametrize("seed,o_range,n", [(45, (0.2, 0.95), 25), (46, (0.6, 1.0), 90)])
def test_backward_with_background_and_dT_matches_central_differences(seed, o_range, n):
    """L = sum g . C + sum gT T_final with C including T_final bg."""
    s, g, W, H = _fd_scene(seed, o_range, n)
    rng = np.random.default_rng(seed + 100)
    bg = rng.uniform(-1, 1, 3).astype(np.float32)
    gT = rng.standard_normal((H, W)).astype(np.float32)
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H, bg=bg)
    grads = oracle.render_bwd(s, si, r, W, H, f["last"], g, bg=bg, dL_dT=gT)
    base = s.astype(np.float64)
    g64, gT64 = g.astype(np.float64), gT.astype(np.float64)
    fd = np.zeros_like(grads)
    for i in range(len(s)):
        for j in range(9):
            h = 1e-6 * max(1.0, abs(base[i, j]))
            vals = []
            for sign in (1, -1):
                v = base.copy()
                v[i, j] += sign * h
                rgb, T = oracle.render_fwd_values(s, v, si, r, W, H, f["last"], bg=bg)
                vals.append(float((rgb * g64).sum() + (T * gT64).sum()))
            fd[i, j] = (vals[0] - vals[1]) / (2 * h)
    scale = np.abs(grads).max(axis=0) + 1e-12
    err = np.abs(fd - grads) / scale
    assert err.max() < 1e-6, (err.max(axis=0))
    # the extra terms change the gradient: without them the FD check would fail
    plain = oracle.render_bwd(s, si, r, W, H, f["last"], g)
    assert np.abs(plain - grads).max() > 1e-3 * np.abs(grads).max()


def test_background_acts_as_a_transmittance_gradient():
    """T_final bg . g enters L like T_final with weight bg . g, so a background
    equals an extra dL/dT_final of bg . g (up to the fp32 rounding of that sum)."""
    s, g, W, H = _fd_scene(47)
    bg = np.array([0.5, -0.25, 0.75], np.float32)
    si, r = _frame_from_splats(s, W, H)
    f = oracle.render_fwd(s, si, r, W, H, bg=bg)
    G1 = oracle.render_bwd(s, si, r, W, H, f["last"], g, bg=bg)
    dT = np.einsum("c,chw->hw", bg.astype(np.float64), g.astype(np.float64)).astype(np.float32)
    G2 = oracle.render_bwd(s, si, r, W, H, f["last"], g, dL_dT=dT)
    np.testing.assert_allclose(G1, G2, rtol=1e-6, atol=1e-9 * np.abs(G1).max())
