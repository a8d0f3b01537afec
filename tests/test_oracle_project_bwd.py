"""Pins of the oracle's projection backward (the chain from the 9 screen-space
gradients to the per-Gaussian ones) against central finite differences of the
oracle's fp64 forward projection, and of its Cartesian SH table against the
Legendre-based basis (not against the backward itself).

Projection: "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on
GPUs", section 2.1, Eq. 1. SH colour and its gradient dL/ds_k = Y_k(d) dL/dc:
"What the 3DGS Literature Left on the Table", Step 3.
"""
import numpy as np

import oracle
import scenegen


def _rot(q):
    w, x, y, z = q / np.linalg.norm(q)
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                     [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                     [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def _scene(seed=5, n=40, degree=3):
    """Visible, well-conditioned Gaussians seen through a rotated, translated camera."""
    rng = np.random.default_rng(seed)
    R = _rot(np.array([1.0, 0.15, -0.1, 0.05]))
    t = np.array([0.3, -0.2, 0.5])
    cam = scenegen.pinhole(96, 80, 90.0, np.concatenate([R, t[:, None]], 1))
    cam.lowpass = 0.3
    # camera-space points in front of the camera, mapped back to world space
    pc = np.stack([rng.uniform(-0.8, 0.8, n), rng.uniform(-0.6, 0.6, n), rng.uniform(2.0, 5.0, n)], 1)
    means = (pc - t) @ R                      # R^T (p - t)
    log_scales = rng.normal(-2.5, 0.4, (n, 3))
    quats = rng.normal(0, 1, (n, 4))
    opac = rng.uniform(0.2, 0.95, n)
    sh = rng.normal(0, 0.3, (n, (degree + 1) ** 2, 3))
    arrs = [a.astype(np.float32) for a in (means, log_scales, quats, opac, sh)]
    return arrs, cam, degree


def test_sh_cartesian_table_equals_legendre_basis():
    rng = np.random.default_rng(1)
    for _ in range(50):
        d = rng.normal(size=3)
        d /= np.linalg.norm(d)
        Y, _ = oracle.sh_cart(3, d)
        assert np.allclose(Y, oracle.sh_basis(3, d), rtol=1e-12, atol=1e-14)


def test_sh_cartesian_gradient_is_the_tangent_derivative():
    rng = np.random.default_rng(2)
    h = 1e-6
    for _ in range(30):
        d = rng.normal(size=3)
        d /= np.linalg.norm(d)
        e = rng.normal(size=3)
        e -= d * (d @ e)
        e /= np.linalg.norm(e)
        _, dY = oracle.sh_cart(3, d)
        fp = oracle.sh_basis(3, (d + h * e) / np.linalg.norm(d + h * e))
        fm = oracle.sh_basis(3, (d - h * e) / np.linalg.norm(d - h * e))
        assert np.allclose(dY @ e, (fp - fm) / (2 * h), rtol=1e-7, atol=1e-8)


def test_backward_equals_finite_differences_of_the_forward():
    (means, ls, qs, op, sh), cam, deg = _scene()
    n = means.shape[0]
    rng = np.random.default_rng(3)
    g = rng.normal(0, 1, (n, 9))
    rec = oracle.project64(means, ls, qs, op, sh, deg, cam)
    assert np.all(rec[:, 9] > 0)
    ana = oracle.project_bwd(means, ls, qs, op, sh, deg, cam, g)

    inputs = dict(means=means, log_scales=ls, quats=qs, opacities=op, sh=sh)

    def loss(vals):
        r = oracle.project64(vals["means"], vals["log_scales"], vals["quats"], vals["opacities"],
                             vals["sh"], deg, cam)
        return np.sum(r[:, :9] * g, axis=1)     # one value per Gaussian

    for name, arr in inputs.items():
        base = {k: v.astype(np.float64) for k, v in inputs.items()}
        flat = base[name].reshape(n, -1)
        fd = np.zeros_like(flat)
        for j in range(flat.shape[1]):
            h = 1e-6 * np.maximum(1.0, np.abs(flat[:, j]))
            plus = {k: v.copy() for k, v in base.items()}
            minus = {k: v.copy() for k, v in base.items()}
            plus[name].reshape(n, -1)[:, j] += h
            minus[name].reshape(n, -1)[:, j] -= h
            fd[:, j] = (loss(plus) - loss(minus)) / (2 * h)
        a = ana[name].reshape(n, -1)
        err = np.linalg.norm(a - fd) / np.linalg.norm(fd)
        assert err < 1e-6, (name, err)


def test_culled_gaussians_get_zero_gradients():
    (means, ls, qs, op, sh), cam, deg = _scene(seed=6, n=6)
    R = np.asarray(cam.world_to_cam).reshape(3, 4)[:, :3]
    t = np.asarray(cam.world_to_cam).reshape(3, 4)[:, 3]
    means[0] = ((np.array([0.0, 0.0, 0.1]) - t) @ R).astype(np.float32)   # in front of znear only
    means[1] = ((np.array([0.0, 0.0, -2.0]) - t) @ R).astype(np.float32)  # behind the camera
    op[2] = 0.5 / 255.0                                                  # below the alpha cutoff
    qs[3] = 0.0                                                           # no rotation
    g = np.ones((6, 9))
    out = oracle.project_bwd(means, ls, qs, op, sh, deg, cam, g)
    for k, v in out.items():
        assert np.all(v[:4] == 0), k
        assert np.any(v[4:] != 0), k
