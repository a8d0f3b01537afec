"""The seeded synthetic scenes: sizes, value distributions, reproducibility."""
import numpy as np
import pytest

import scenegen


def _logit(o):
    o = o.astype(np.float64)
    return np.log(o / (1 - o))


def test_tiny_and_small_shapes_and_moments():
    t = scenegen.make_config(1)
    assert t.n == 1000 and t.sh.shape == (1000, 1, 3) and t.dL_drgb.shape == (3, 64, 64)
    assert t.camera.num_tiles == 16
    assert np.all(np.abs(t.means[:, :2]) <= 1) and np.all((t.means[:, 2] >= 2) & (t.means[:, 2] <= 4))
    s = scenegen.make_config(2)
    assert s.n == 100_000 and s.sh.shape == (100_000, 16, 3) and s.camera.num_tiles == 256
    assert abs(s.log_scales.mean() + 3.5) < 0.01 and abs(s.log_scales.std() - 0.3) < 0.01
    lg = _logit(s.opacities)
    assert abs(lg.mean()) < 0.02 and abs(lg.std() - 1.0) < 0.02
    assert np.all(np.abs(s.sh[:, 0]) <= 0.5) and abs(s.sh[:, 1:].std() - 0.05) < 0.001
    np.testing.assert_allclose(np.linalg.norm(s.quats, axis=1), 1.0, atol=1e-6)
    assert abs(s.dL_drgb.std() - 1.0) < 0.01


def test_seeded_reproducibility():
    a = scenegen.make_config(2)
    b = scenegen.make_config(2)
    for f in ("means", "log_scales", "quats", "opacities", "sh", "dL_drgb"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = scenegen.make_config(2, seed=7)
    assert not np.array_equal(a.means, c.means)


def test_garden_shape():
    g = scenegen.make_config(3)
    assert g.n == 1_535_033 and g.camera.width == 1297 and g.camera.height == 840
    assert g.camera.num_tiles == 4346
    z = g.means[:, 2]
    assert z.min() >= 1.0 and z.max() <= 20.0
    r = np.linalg.norm(g.means.astype(np.float64), axis=1)
    shell = (r >= 15) & (r <= 20)
    assert shell.sum() >= 307_007      # the shell plus any cluster members at that radius
    lg = _logit(g.opacities)
    assert abs(lg.mean() - 0.5) < 0.01 and abs(lg.std() - 1.5) < 0.01


@pytest.mark.slow
def test_room_and_urban_shapes():
    r = scenegen.make_config(4)
    assert r.n == 3_000_000 and r.camera.num_tiles == 98 * 65
    assert abs((r.log_scales[:, 2] - r.log_scales[:, 0]).mean() + 2.0) < 0.01
    front = (np.abs(r.means[:, 2] - 3.0) < 0.1) & (np.abs(r.means[:, 1]) < 1.4) & (np.abs(r.means[:, 0]) < 2.9)
    assert abs(front.mean() - 0.125 * (2.8 / 3) * (5.8 / 6)) < 0.003
    u = scenegen.make_config(5)
    assert u.n == 6_000_000 and u.camera.num_tiles == 120 * 68
    assert u.means[:, 2].min() >= 2.0 and u.means[:, 2].max() <= 200.0
    lg = _logit(u.opacities)
    assert abs(lg.std() - np.sqrt(2.0)) < 0.01


def test_bf16_rounding_is_ieee_nearest_even():
    # known patterns, the two tie directions, and the carry into the exponent
    x = np.array([1.0, -2.0, 0.5, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20,
                  2 - 2 ** -9, 0.0, -0.0, np.inf, 3.0e38], dtype=np.float32)
    bits, wide = scenegen.to_bf16(x)
    assert list(bits) == [0x3F80, 0xC000, 0x3F00, 0x3F80, 0x3F82, 0x3F81, 0x4000, 0, 0x8000,
                          0x7F80, 0x7F62]
    big = np.array([0x7F620000], dtype=np.uint32).view(np.float32)[0]
    np.testing.assert_array_equal(wide, np.array([1.0, -2.0, 0.5, 1.0, 1 + 2 ** -6, 1 + 2 ** -7,
                                                  2.0, 0.0, -0.0, np.inf, big], dtype=np.float32))
    assert np.signbit(wide[8])
    # within half a bf16 ulp, and the same as torch's conversion on random data
    rng = np.random.default_rng(5)
    y = rng.normal(0, 0.3, 100_000).astype(np.float32)
    b, w = scenegen.to_bf16(y)
    ulp = np.ldexp(1.0, np.frexp(np.abs(y).astype(np.float64))[1] - 8)
    assert np.all(np.abs(w.astype(np.float64) - y) <= 0.5 * ulp)
    torch = pytest.importorskip("torch")
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, tb)
