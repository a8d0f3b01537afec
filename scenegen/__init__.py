"""Seeded synthetic scenes for the Gaussian-splatting rasterizer.

This module only draws random numbers: Gaussian centres, log-scales, rotation
quaternions, opacities, SH coefficients, a pinhole camera and an upstream
image gradient. It holds none of the rendering method's arithmetic, so that the
CPU oracle and the HIP path can both take their inputs from it.

The pages measure trained scenes (Mip-NeRF 360 garden and room, urban and
driving captures). Those datasets are not available here; each scene below is
a synthetic stand-in with the stated size, image shape and value
distributions. The five configurations are:

1. tiny    1,000 Gaussians, 64x64, SH degree 0
2. small   100,000 Gaussians, 256x256, SH degree 3
3. garden  1,535,033 Gaussians, 1297x840, SH degree 3 (the shape of the
           Metal trainer's garden run on the msplat pull-request page)
4. room    3,000,000 Gaussians, 1557x1038, SH degree 3
5. urban   6,000,000 Gaussians, 1920x1080, SH degree 3, heavy-tile skew

Random streams: numpy PCG64 seeded with ``20261202 + config``;
``SeedSequence(seed).spawn(8)`` gives, in order, the streams for means,
log-scales, quaternions, opacity, SH DC, SH rest, cluster parameters and the
upstream gradient. N(mu, s^2) always means variance s^2.
"""
from __future__ import annotations

import dataclasses
import numpy as np

BASE_SEED = 20261202

CONFIG_NAMES = {1: "tiny", 2: "small", 3: "garden", 4: "room", 5: "urban"}


@dataclasses.dataclass
class Camera:
    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    world_to_cam: np.ndarray  # float32[12], row-major [R|t]
    znear: float = 0.2
    lowpass: float = 0.3

    @property
    def tiles_x(self) -> int:
        return (self.width + 15) // 16

    @property
    def tiles_y(self) -> int:
        return (self.height + 15) // 16

    @property
    def num_tiles(self) -> int:
        return self.tiles_x * self.tiles_y


@dataclasses.dataclass
class Scene:
    name: str
    means: np.ndarray        # float32[N,3]
    log_scales: np.ndarray   # float32[N,3]
    quats: np.ndarray        # float32[N,4]  (w, x, y, z), not necessarily unit
    opacities: np.ndarray    # float32[N]    activated, in (0, 1)
    sh: np.ndarray           # float32[N,K,3]
    sh_degree: int
    camera: Camera
    dL_drgb: np.ndarray      # float32[3,H,W]

    @property
    def n(self) -> int:
        return int(self.means.shape[0])


def pinhole(width: int, height: int, f: float, world_to_cam=None,
            znear: float = 0.2, lowpass: float = 0.3) -> Camera:
    """A pinhole camera with the principal point at the image centre."""
    if world_to_cam is None:
        world_to_cam = np.array([1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 0], np.float32)
    return Camera(int(width), int(height), float(f), float(f), width / 2.0,
                  height / 2.0, np.asarray(world_to_cam, np.float32).reshape(12),
                  float(znear), float(lowpass))


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(8)]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_quats(rng, n):
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    return q


def _sh(rng_dc, rng_rest, n, degree):
    k = (degree + 1) ** 2
    sh = np.empty((n, k, 3), np.float32)
    sh[:, 0, :] = rng_dc.uniform(-0.5, 0.5, (n, 3))
    if k > 1:
        rest = rng_rest.standard_normal((n, k - 1, 3), dtype=np.float32)
        rest *= np.float32(0.05)
        sh[:, 1:, :] = rest
    return sh


def _random_rotation(rng):
    """Uniform random 3x3 rotation from the QR factorisation of a Gaussian matrix."""
    a = rng.standard_normal((3, 3))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def _largest_remainder(weights, total, minimum=1):
    k = len(weights)
    rest = total - minimum * k
    share = weights / weights.sum() * rest
    counts = np.floor(share).astype(np.int64)
    left = rest - int(counts.sum())
    order = np.argsort(-(share - counts), kind="stable")
    counts[order[:left]] += 1
    return counts + minimum


def _fill(rng, n, draw, accept):
    """Rejection sampling: draw(rng, m) -> [m,3]; keep rows with accept(rows)."""
    out = np.empty((0, 3))
    while out.shape[0] < n:
        m = max(1024, int((n - out.shape[0]) * 1.3))
        cand = draw(rng, m)
        out = np.concatenate([out, cand[accept(cand)]])
    return out[:n]


def _finish(name, seed_streams, means, log_scale_mu, log_scale_sd, op_mu, op_sd,
            degree, cam, flatten_third=False):
    r_means, r_scales, r_quats, r_op, r_dc, r_rest, _r_cl, r_grad = seed_streams
    n = means.shape[0]
    ls = r_scales.normal(log_scale_mu, log_scale_sd, (n, 3))
    if flatten_third:
        ls[:, 2] -= 2.0
    quats = _unit_quats(r_quats, n)
    opac = _sigmoid(r_op.normal(op_mu, op_sd, n))
    sh = _sh(r_dc, r_rest, n, degree)
    grad = r_grad.standard_normal((3, cam.height, cam.width), dtype=np.float32)
    return Scene(name, means.astype(np.float32), ls.astype(np.float32),
                 quats.astype(np.float32), opac.astype(np.float32), sh, degree,
                 cam, grad.astype(np.float32))


def make_tiny(seed=BASE_SEED + 1):
    st = _streams(seed)
    n = 1000
    m = np.stack([st[0].uniform(-1, 1, n), st[0].uniform(-1, 1, n),
                  st[0].uniform(2, 4, n)], 1)
    return _finish("tiny", st, m, -3.5, 0.3, 0.0, 1.0, 0, pinhole(64, 64, 64.0))


def make_small(seed=BASE_SEED + 2):
    st = _streams(seed)
    n = 100_000
    m = np.stack([st[0].uniform(-2, 2, n), st[0].uniform(-2, 2, n),
                  st[0].uniform(2, 8, n)], 1)
    return _finish("small", st, m, -3.5, 0.3, 0.0, 1.0, 3, pinhole(256, 256, 256.0))


def make_garden(seed=BASE_SEED + 3):
    """64 anisotropic clusters (80%) plus a uniform background shell (20%)."""
    st = _streams(seed)
    rm, rc = st[0], st[6]
    n_total, n_cluster = 1_535_033, 1_228_026
    n_shell = n_total - n_cluster
    w, h, f = 1297, 840, 1100.0
    weights = rc.dirichlet(np.ones(64))
    counts = rc.multinomial(n_cluster, weights)
    parts = []
    in_depth = lambda p: (p[:, 2] >= 1.0) & (p[:, 2] <= 20.0)
    for ci in range(64):
        zc = rc.uniform(2, 18)
        xc = zc * rc.uniform(-0.9, 0.9) * w / (2 * f)
        yc = zc * rc.uniform(-0.9, 0.9) * h / (2 * f)
        sig = zc * rc.uniform(0.02, 0.12, 3)
        rot = _random_rotation(rc)
        chol = rot * sig  # columns scaled: cov = rot diag(sig^2) rot^T
        centre = np.array([xc, yc, zc])
        cnt = int(counts[ci])
        if cnt == 0:
            continue
        draw = lambda g, m_, c=centre, L=chol: c + g.standard_normal((m_, 3)) @ L.T
        parts.append(_fill(rm, cnt, draw, in_depth))

    def shell(g, m_):
        r = np.cbrt(15.0 ** 3 + g.uniform(0, 1, m_) * (20.0 ** 3 - 15.0 ** 3))
        d = g.standard_normal((m_, 3))
        d /= np.linalg.norm(d, axis=1, keepdims=True)
        return d * r[:, None]

    parts.append(_fill(rm, n_shell, shell, in_depth))
    means = np.concatenate(parts)
    return _finish("garden", st, means, -4.0, 0.6, 0.5, 1.5, 3, pinhole(w, h, f))


def make_room(seed=BASE_SEED + 4):
    """Six walls of a 6x3x6 m box (y down), camera at the centre."""
    st = _streams(seed)
    rm, rc = st[0], st[6]
    n = 3_000_000
    # floor, ceiling 25% each; four walls 12.5% each (shares proportional to area)
    counts = _largest_remainder(np.array([2, 2, 1, 1, 1, 1], float), n, 0)
    parts = []
    for wall, cnt in enumerate(counts):
        u = rm.uniform(0, 1, (cnt, 2))
        off = rm.normal(0.0, 0.02, cnt)
        p = np.empty((cnt, 3))
        if wall in (0, 1):   # floor y=+1.5, ceiling y=-1.5
            p[:, 0] = -3 + 6 * u[:, 0]
            p[:, 2] = -3 + 6 * u[:, 1]
            p[:, 1] = (1.5 if wall == 0 else -1.5) + off
        elif wall in (2, 3):  # walls z=+3, z=-3
            p[:, 0] = -3 + 6 * u[:, 0]
            p[:, 1] = -1.5 + 3 * u[:, 1]
            p[:, 2] = (3.0 if wall == 2 else -3.0) + off
        else:                 # walls x=+3, x=-3
            p[:, 2] = -3 + 6 * u[:, 0]
            p[:, 1] = -1.5 + 3 * u[:, 1]
            p[:, 0] = (3.0 if wall == 4 else -3.0) + off
        parts.append(p)
    means = np.concatenate(parts)
    return _finish("room", st, means, -4.5, 0.5, 1.0, 1.0, 3,
                   pinhole(1557, 1038, 1200.0), flatten_third=True)


def make_urban(seed=BASE_SEED + 5):
    """2,000 Pareto-sized clusters along a street corridor, depth 2..200."""
    st = _streams(seed)
    rm, rc = st[0], st[6]
    n, k = 6_000_000, 2000
    sizes = rc.pareto(1.2, k) + 1.0          # Pareto I, x_m = 1
    counts = _largest_remainder(sizes, n, 1)
    zc = rc.uniform(2, 200, k)
    kind = rc.choice(3, size=k, p=[0.4, 0.4, 0.2])
    xc = np.where(kind == 0, -8 + rc.standard_normal(k),
                  np.where(kind == 1, 8 + rc.standard_normal(k), rc.uniform(-8, 8, k)))
    yc = np.where(kind == 2, 1.5 + rc.normal(0, 0.05, k), rc.uniform(-10, 1.5, k))
    centres = np.stack([xc, yc, zc], 1)
    in_depth = lambda p: (p[:, 2] >= 2.0) & (p[:, 2] <= 200.0)
    parts = []
    for ci in range(k):
        c = centres[ci]
        draw = lambda g, m_, c=c: c + 0.5 * g.standard_normal((m_, 3))
        parts.append(_fill(rm, int(counts[ci]), draw, in_depth))
    means = np.concatenate(parts)
    return _finish("urban", st, means, -4.0, 0.8, 0.0, np.sqrt(2.0), 3,
                   pinhole(1920, 1080, 1400.0))


MAKERS = {1: make_tiny, 2: make_small, 3: make_garden, 4: make_room, 5: make_urban}


def make_config(i: int, seed: int | None = None) -> Scene:
    """Scene for configuration i (1..5) with its default seed 20261202 + i."""
    maker = MAKERS[int(i)]
    return maker() if seed is None else maker(seed)


def random_scene(seed: int, n: int, width: int, height: int, f: float,
                 degree: int = 0, depth=(2.0, 6.0), spread=1.0,
                 log_scale=(-3.0, 0.5), opacity=(0.0, 1.5)) -> Scene:
    """A small seeded scene for unit tests (ragged sizes, any degree)."""
    st = _streams(seed)
    rm = st[0]
    z = rm.uniform(depth[0], depth[1], n)
    hx = spread * width / (2 * f)
    hy = spread * height / (2 * f)
    m = np.stack([z * rm.uniform(-hx, hx, n), z * rm.uniform(-hy, hy, n), z], 1)
    cam = pinhole(width, height, f)
    return _finish(f"random{seed}", st, m, log_scale[0], log_scale[1],
                   opacity[0], opacity[1], degree, cam)


def to_bf16(x):
    """Round fp32 values to bfloat16, nearest with ties to even (the IEEE rule):
    returns the 16-bit patterns (uint16, the upper half of the fp32 word) and
    the same values widened back to fp32 exactly. NaNs keep a set quiet bit."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = np.where(nan, (u >> 16) | 0x40, r).astype(np.uint16)
    wide = (r.astype(np.uint32) << 16).view(np.float32)
    return r.reshape(np.shape(x)), wide.reshape(np.shape(x))
