"""The raster kernels' sub-tile cull and forward-state layout, run on the CPU.

"What the 3DGS Literature Left on the Table", Step 1 (c): a staged batch of
splats is culled against each wavefront's part of the tile, and Step 5: the
hit decision is the canonical fp32 q <= tau. The cull may keep sub-tiles
without a hit, but must never drop one that holds a hit pixel, or the forward
pass would lose that blend. The check compiles the kernels' own header
(csrc/cull.h) for the host and runs it over every 8x8 sub-tile of random,
needle-thin (anisotropy above 1e3), screen-sized and off-screen-centred splat
records, including records whose cutoff passes exactly through a pixel centre.
"""
import ctypes as C
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gaussian_splatting_differentiable_amd", "csrc")


@pytest.fixture(scope="module")
def cull():
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp(prefix="hostchk")
    so = os.path.join(d, "host_checks.so")
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "host_checks.hip"), "-o", so]
    subprocess.run(cmd, check=True, capture_output=True)
    L = C.CDLL(so)
    L.cull_check.argtypes = [C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
    L.cull_check.restype = None
    L.state_bytes.argtypes, L.state_bytes.restype = [C.c_int, C.c_int64], C.c_int64
    L.state_capacity.argtypes, L.state_capacity.restype = [C.c_int, C.c_int64], C.c_int64
    yield L
    shutil.rmtree(d, ignore_errors=True)


def _records(rng, n, W, H, lam_thin, lam_long, far):
    """Screen-space records with covariance eigenvalues (lam_thin, lam_long) px^2
    at a random angle, centres up to `far` px outside the image."""
    th = rng.uniform(0, np.pi, n)
    l1, l2 = lam_thin(n), lam_long(n)
    cs, sn = np.cos(th), np.sin(th)
    sxx, syy, sxy = cs * cs * l1 + sn * sn * l2, sn * sn * l1 + cs * cs * l2, cs * sn * (l1 - l2)
    det = sxx * syy - sxy * sxy
    rec = np.zeros((n, 12), np.float32)
    rec[:, 0] = rng.uniform(-far, W + far, n)
    rec[:, 1] = rng.uniform(-far, H + far, n)
    rec[:, 2], rec[:, 3], rec[:, 4] = syy / det, -sxy / det, sxx / det
    o = np.clip(1 / (1 + np.exp(-rng.normal(0, 2, n))), 0.005, 0.999)
    rec[:, 5] = o
    rec[:, 9] = (2 * np.log(255 * o)).astype(np.float32)
    return rec


def _fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) +
            np.asarray(c, np.float64)).astype(np.float32)


def _canon_q(rec, px, py):
    dx = (np.float32(px) + np.float32(0.5)) - rec[:, 0]
    dy = (np.float32(py) + np.float32(0.5)) - rec[:, 1]
    return _fma32(rec[:, 4] * dy, dy, _fma32(np.float32(2) * rec[:, 3] * dx, dy, (rec[:, 2] * dx) * dx))


def _run(L, rec, W, H):
    out = np.zeros(3, np.int64)
    rec = np.ascontiguousarray(rec, np.float32)
    L.cull_check(len(rec), rec.ctypes.data, W, H, out.ctypes.data)
    return out


W, H = 320, 240
CASES = {
    # eigenvalues in px^2 (the EWA low-pass keeps the thin one at 0.3 or more)
    "random": (lambda r, n: 0.3 + np.exp(r.normal(1, 1.5, n)),
               lambda r, n: 0.3 + np.exp(r.normal(1, 1.5, n)), 50, 4000),
    "needle": (lambda r, n: 0.3 + r.uniform(0, 0.05, n),
               lambda r, n: np.exp(r.uniform(np.log(300), np.log(3e5), n)), 50, 3000),
    "screen": (lambda r, n: np.exp(r.uniform(np.log(1e3), np.log(1e5), n)),
               lambda r, n: np.exp(r.uniform(np.log(1e3), np.log(1e6), n)), 50, 300),
    "needle_far": (lambda r, n: 0.3 + r.uniform(0, 0.02, n),
                   lambda r, n: np.exp(r.uniform(np.log(1e5), np.log(1e8), n)), 2000, 400),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_cull_keeps_every_hit_subtile(cull, case):
    lam1, lam2, far, n = CASES[case]
    rng = np.random.default_rng(7 + sorted(CASES).index(case))
    rec = _records(rng, n, W, H, lambda k: lam1(rng, k), lambda k: lam2(rng, k), far)
    missed, with_hit, extra = _run(cull, rec, W, H)
    assert with_hit > 200
    assert missed == 0, (case, missed, with_hit)
    # still a cull: a few extra sub-tiles, more only where the guard scales with
    # the large terms of a far, long splat
    assert extra < (0.5 if case == "needle_far" else 0.05) * with_hit + 50


@pytest.mark.parametrize("case,far", [("random", 50), ("needle", 2000), ("screen", 3000)])
def test_cull_with_the_cutoff_through_a_pixel(cull, case, far):
    """Records whose cutoff tau equals the canonical q at one pixel centre: that
    pixel is a hit with q == tau exactly, the tightest case for the guard. The
    long, thin, tilted splats centred far off screen are where the terms of q
    cancel most (a guard proportional to tau alone missed 21 such sub-tiles
    here)."""
    lam1, lam2, _, _ = CASES[case]
    rng = np.random.default_rng({"random": 11, "needle": 12, "screen": 13}[case])
    hi = {"needle": 1e7, "screen": 1e7}.get(case)
    total_hits = 0
    for rep in range(12):
        n = 20000 if case != "screen" else 2000
        long_ = (lambda k: np.exp(rng.uniform(np.log(300), np.log(hi), k))) if case == "needle" \
            else (lambda k: lam2(rng, k))
        rec = _records(rng, n, W, H, lambda k: lam1(rng, k), long_, far)
        px, py = rng.integers(0, W, n), rng.integers(0, H, n)
        q = _canon_q(rec, px, py)
        ok = (q > 0) & (q < np.float32(2 * np.log(255.0)))
        rec = rec[ok]
        rec[:, 9] = q[ok]
        missed, with_hit, _ = _run(cull, rec, W, H)
        assert missed == 0, (case, rep, missed)
        total_hits += with_hit
    assert total_hits > 1000


@pytest.mark.parametrize("T", [1, 16, 4346, 8160, 65535])
def test_forward_state_serves_the_capacity_it_was_sized_for(cull, T):
    """A forward state of gs_fwd_state_size(W, H, cap) bytes holds the
    contributor record of any frame of up to cap pairs (the forward refuses a
    frame with more pairs than the state serves), for capacities that are and
    are not multiples of the 64-entry batch."""
    L = cull
    base = L.state_bytes(T, 0)
    assert L.state_capacity(T, base - 1) == -1
    for cap in [0, 1, 63, 64, 65, 4095, 7_913_276, 9_033_723, (1 << 30) - 1]:
        b = L.state_bytes(T, cap)
        assert b % 256 == 0 and b >= base
        got = L.state_capacity(T, b)
        assert cap <= got < cap + 64 * 9, (T, cap, got)
