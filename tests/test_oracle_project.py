"""Pins of the oracle's projection and SH colour against closed forms,
library routines and invariances (not against the oracle itself).

Projection: "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on
GPUs", section 2.1, Eq. 1. SH colour: "What the 3DGS Literature Left on the
Table", Step 3 (colour = sum_k Y_k(d) s_k over 16 basis functions).
"""
import math

import numpy as np
import pytest
from scipy import special

import oracle
import scenegen


def _cam(w=64, h=48, f=50.0, fy=None, w2c=None):
    c = scenegen.pinhole(w, h, f, w2c)
    if fy is not None:
        c.fy = fy
    return c


def _one(mean, log_scale, quat, opacity, cam, sh=None, degree=0):
    if sh is None:
        sh = np.zeros((1, (degree + 1) ** 2, 3), np.float32)
        sh[0, 0] = [0.1, 0.2, 0.3]
    _, rec = oracle.project(np.array([mean], np.float32), np.array([log_scale], np.float32),
                            np.array([quat], np.float32), np.array([opacity], np.float32),
                            sh, degree, cam, want_f64=True)
    return rec[0]


def _conic_to_cov(rec):
    a, b, c = rec[2], rec[3], rec[4]
    return np.linalg.inv(np.array([[a, b], [b, c]]))


# ---------------------------------------------------------------- SH basis

def test_sh_y00_value():
    for d in ([0, 0, 1], [1, 0, 0], [0.6, 0.0, 0.8]):
        assert oracle.sh_basis(0, d)[0] == pytest.approx(1.0 / (2.0 * math.sqrt(math.pi)), abs=1e-15)


def test_sh_degree1_is_y_z_x():
    rng = np.random.default_rng(0)
    for _ in range(10):
        d = rng.standard_normal(3)
        d /= np.linalg.norm(d)
        Y = oracle.sh_basis(1, d)
        np.testing.assert_allclose(Y[1:4], math.sqrt(3 / (4 * math.pi)) * d[[1, 2, 0]], atol=1e-14)


def test_sh_matches_scipy_complex_harmonics():
    """Real SH without Condon-Shortley phase from scipy's complex Y_l^m (which
    carries the phase): m>0: sqrt2 (-1)^m Re Y_l^m; m<0: sqrt2 (-1)^m Im Y_l^|m|."""
    rng = np.random.default_rng(1)
    for _ in range(20):
        d = rng.standard_normal(3)
        d /= np.linalg.norm(d)
        theta = math.acos(d[2])
        phi = math.atan2(d[1], d[0])
        Y = oracle.sh_basis(3, d)
        for l in range(4):
            for m in range(-l, l + 1):
                am = abs(m)
                yc = special.sph_harm_y(l, am, theta, phi)
                if m > 0:
                    ref = math.sqrt(2) * (-1) ** am * yc.real
                elif m < 0:
                    ref = math.sqrt(2) * (-1) ** am * yc.imag
                else:
                    ref = yc.real
                assert Y[l * (l + 1) + m] == pytest.approx(ref, abs=1e-12), (l, m)


def test_sh_orthonormal_by_quadrature():
    x, wx = np.polynomial.legendre.leggauss(16)   # exact for polynomials in cos(theta)
    nphi = 32
    phis = 2 * np.pi * np.arange(nphi) / nphi
    gram = np.zeros((16, 16))
    for ct, w in zip(x, wx):
        st = math.sqrt(1 - ct * ct)
        for ph in phis:
            Y = oracle.sh_basis(3, [st * math.cos(ph), st * math.sin(ph), ct])
            gram += np.outer(Y, Y) * w * (2 * np.pi / nphi)
    np.testing.assert_allclose(gram, np.eye(16), atol=1e-10)


# ---------------------------------------------------------------- projection closed forms

def test_isotropic_on_axis():
    cam = _cam()
    Z, sig, o = 3.0, 0.05, 0.7
    rec = _one([0, 0, Z], [math.log(sig)] * 3, [0.3, -0.5, 0.1, 0.8], o, cam)
    var = (cam.fx * sig / Z) ** 2 + cam.lowpass
    assert rec[0] == pytest.approx(cam.cx) and rec[1] == pytest.approx(cam.cy)
    np.testing.assert_allclose(rec[2:5], [1 / var, 0, 1 / var], rtol=1e-6, atol=1e-9)
    assert rec[5] == pytest.approx(o, rel=1e-7)
    assert rec[9] == pytest.approx(2 * math.log(255 * o), rel=1e-7)
    assert rec[10] == pytest.approx(Z)


def test_axis_aligned_anisotropic():
    cam = _cam(fy=80.0)
    Z, s = 4.0, np.array([0.03, 0.11, 0.07])
    rec = _one([0, 0, Z], np.log(s), [1, 0, 0, 0], 0.5, cam)
    cov = _conic_to_cov(rec)
    np.testing.assert_allclose(cov, np.diag([(cam.fx * s[0] / Z) ** 2 + cam.lowpass,
                                             (cam.fy * s[1] / Z) ** 2 + cam.lowpass]),
                               rtol=1e-6, atol=1e-9)


def test_quaternion_rotations():
    """90 deg about z swaps the x/y scales; 90 deg about x brings the z scale
    onto the image y axis; 30 deg about z tilts the major axis toward +y."""
    cam = _cam()
    Z, s = 4.0, np.array([0.03, 0.11, 0.07])
    f2 = (cam.fx / Z) ** 2
    h = math.sqrt(0.5)
    cov = _conic_to_cov(_one([0, 0, Z], np.log(s), [h, 0, 0, h], 0.5, cam))
    np.testing.assert_allclose(cov, np.diag(f2 * s[[1, 0]] ** 2 + cam.lowpass), rtol=1e-6, atol=1e-9)
    cov = _conic_to_cov(_one([0, 0, Z], np.log(s), [h, h, 0, 0], 0.5, cam))
    np.testing.assert_allclose(cov, np.diag(f2 * s[[0, 2]] ** 2 + cam.lowpass), rtol=1e-6, atol=1e-9)
    th = math.radians(30)
    cov = _conic_to_cov(_one([0, 0, Z], np.log(s), [math.cos(th / 2), 0, 0, math.sin(th / 2)], 0.5, cam))
    R2 = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
    ref = f2 * R2 @ np.diag(s[:2] ** 2) @ R2.T + cam.lowpass * np.eye(2)
    np.testing.assert_allclose(cov, ref, rtol=1e-6, atol=1e-9)
    assert cov[0, 1] < 0  # sx < sy: rotating +30 deg puts the long axis at 120 deg


def test_off_axis_isotropic_is_s2_JJt():
    cam = _cam(fy=70.0)
    X, Y, Z, sig = 0.7, -0.4, 2.5, 0.04
    rec = _one([X, Y, Z], [math.log(sig)] * 3, [0.2, 0.4, -0.3, 0.5], 0.9, cam)
    jjt = np.array([[cam.fx ** 2 * (1 / Z ** 2 + X ** 2 / Z ** 4), cam.fx * cam.fy * X * Y / Z ** 4],
                    [cam.fx * cam.fy * X * Y / Z ** 4, cam.fy ** 2 * (1 / Z ** 2 + Y ** 2 / Z ** 4)]])
    np.testing.assert_allclose(_conic_to_cov(rec), sig ** 2 * jjt + cam.lowpass * np.eye(2),
                               rtol=1e-6, atol=1e-9)
    assert rec[0] == pytest.approx(cam.fx * X / Z + cam.cx)
    assert rec[1] == pytest.approx(cam.fy * Y / Z + cam.cy)


def _quat_mul(a, b):
    w1, x1, y1, z1 = a
    w2, x2, y2, z2 = b
    return np.array([w1 * w2 - x1 * x2 - y1 * y2 - z1 * z2, w1 * x2 + x1 * w2 + y1 * z2 - z1 * y2,
                     w1 * y2 - x1 * z2 + y1 * w2 + z1 * x2, w1 * z2 + x1 * y2 - y1 * x2 + z1 * w2])


def _quat_to_mat(q):
    # rotation of a vector v by q: v' = q v q*; read off by rotating the basis vectors
    cols = []
    for e in np.eye(3):
        v = _quat_mul(_quat_mul(q, np.concatenate([[0.0], e])), q * np.array([1, -1, -1, -1]))
        cols.append(v[1:])
    return np.stack(cols, 1)


def test_rigid_motion_invariance_and_quaternion_scale_sign():
    sc = scenegen.random_scene(5, 200, 80, 60, 60.0, degree=3)
    base = oracle.project_scene(sc, want_f64=True)[1]
    # q -> -q and q -> 2q describe the same rotation
    for fac in (-1.0, 2.0):
        rec = oracle.project(sc.means, sc.log_scales, sc.quats * fac, sc.opacities, sc.sh, 3,
                             sc.camera, want_f64=True)[1]
        np.testing.assert_allclose(rec, base, rtol=1e-9, atol=1e-9)
    # move the world by M and the camera by M^-1
    qm = np.array([0.9, 0.2, -0.3, 0.25])
    qm /= np.linalg.norm(qm)
    Rm = _quat_to_mat(qm)
    tm = np.array([0.3, -1.0, 2.0])
    means2 = (sc.means.astype(np.float64) @ Rm.T + tm)
    quats2 = np.array([_quat_mul(qm, q) for q in sc.quats.astype(np.float64)])
    w2c = np.zeros((3, 4))
    w2c[:, :3] = Rm.T
    w2c[:, 3] = -Rm.T @ tm
    cam2 = scenegen.pinhole(80, 60, 60.0, w2c.reshape(12))
    # the oracle reads float32 inputs; compare the fp64 records loosely
    rec = oracle.project(means2, sc.log_scales, quats2, sc.opacities, sc.sh, 3, cam2, want_f64=True)[1]
    vis = base[:, 9] > 0
    assert np.array_equal(vis, rec[:, 9] > 0)
    np.testing.assert_allclose(rec[vis][:, [0, 1, 10]], base[vis][:, [0, 1, 10]], rtol=2e-5, atol=2e-4)
    np.testing.assert_allclose(rec[vis][:, 2:5], base[vis][:, 2:5], rtol=2e-4, atol=1e-7)
    # SH coefficients live in the world frame: colour is invariant under a pure translation
    w2c_t = np.array([1, 0, 0, -tm[0], 0, 1, 0, -tm[1], 0, 0, 1, -tm[2]])
    rec_t = oracle.project(sc.means.astype(np.float64) + tm, sc.log_scales, sc.quats, sc.opacities,
                           sc.sh, 3, scenegen.pinhole(80, 60, 60.0, w2c_t), want_f64=True)[1]
    np.testing.assert_allclose(rec_t[vis][:, 6:9], base[vis][:, 6:9], rtol=1e-4, atol=1e-5)


def test_culling_rules():
    cam = _cam()
    assert _one([0, 0, 0.19], [-3] * 3, [1, 0, 0, 0], 0.5, cam)[9] == -1      # behind near plane
    assert _one([0, 0, -2.0], [-3] * 3, [1, 0, 0, 0], 0.5, cam)[9] == -1      # behind camera
    assert _one([0, 0, 2.0], [-3] * 3, [1, 0, 0, 0], 0.0039, cam)[9] == -1  # o < 1/255: alpha < 1/255 everywhere
    assert 0 < _one([0, 0, 2.0], [-3] * 3, [1, 0, 0, 0], 0.0040, cam)[9] < 0.05
    rec = _one([0, 0, 2.0], [-3] * 3, [1, 0, 0, 0], 1.0, cam)
    assert rec[9] == pytest.approx(2 * math.log(255.0))
    rec = _one([5.0, 0, 2.0], [-3] * 3, [1, 0, 0, 0], 0.5, cam)              # off-screen: kept
    assert rec[9] > 0


def test_sh_colour_view_direction_and_camera_centre():
    # degree 1, only the x-coefficient: colour = sqrt(3/4pi) * d_x, d from the camera centre
    sh = np.zeros((1, 4, 3), np.float32)
    sh[0, 3] = [1.0, 2.0, -1.0]
    k1 = math.sqrt(3 / (4 * math.pi))
    rec = _one([1.0, 0.0, 1.0], [-3] * 3, [1, 0, 0, 0], 0.5, _cam(), sh=sh, degree=1)
    np.testing.assert_allclose(rec[6:9], k1 * math.sqrt(0.5) * np.array([1.0, 2.0, -1.0]), rtol=1e-6)
    # camera translated by +1 along x (world_to_cam t = -1): camera centre at x = 1
    w2c = [1, 0, 0, -1.0, 0, 1, 0, 0, 0, 0, 1, 0]
    rec = _one([1.0, 0.0, 1.0], [-3] * 3, [1, 0, 0, 0], 0.5, _cam(w2c=w2c), sh=sh, degree=1)
    np.testing.assert_allclose(rec[6:9], [0, 0, 0], atol=1e-7)
    # degree 0: colour does not depend on the view
    sh0 = np.zeros((1, 1, 3), np.float32)
    sh0[0, 0] = [0.4, -0.2, 0.1]
    y00 = 1 / (2 * math.sqrt(math.pi))
    for m in ([0.3, 0.2, 2.0], [-1.0, 0.5, 3.0]):
        rec = _one(m, [-3] * 3, [1, 0, 0, 0], 0.5, _cam(), sh=sh0, degree=0)
        np.testing.assert_allclose(rec[6:9], y00 * np.array([0.4, -0.2, 0.1]), rtol=1e-6)


def test_conic_inverts_covariance_of_random_scene():
    sc = scenegen.random_scene(9, 300, 96, 64, 70.0, degree=2)
    rec = oracle.project_scene(sc, want_f64=True)[1]
    vis = rec[:, 9] > 0
    a, b, c = rec[vis, 2], rec[vis, 3], rec[vis, 4]
    # conic is symmetric positive definite and its inverse has eigenvalues >= lowpass
    det = a * c - b * b
    assert np.all(a > 0) and np.all(c > 0) and np.all(det > 0)
    lam_max_conic = 0.5 * (a + c) + np.sqrt(0.25 * (a - c) ** 2 + b * b)
    assert np.all(lam_max_conic <= 1 / sc.camera.lowpass * (1 + 1e-9))
