"""SH coefficients stored as bfloat16 (gs_project_bf16sh, gs_project_bwd_bf16sh).

"What the 3DGS Literature Left on the Table", Step 3 and Step 6: the SH
parameters are kept in bf16 to halve their bytes; the arithmetic stays fp32.
The kernels widen each bf16 value exactly, so the bf16 calls must give, bit for
bit, what the fp32 calls give on the widened coefficients; and the oracle, run
on the same bf16-rounded values, bounds both with the unchanged parity rules.
The SH rows are placed at the weakest alignment each degree allows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import scenegen
from test_gpu_parity import check_projection
from test_gpu_project_bwd import _check

pytestmark = pytest.mark.gpu

# weakest allowed alignment of the bf16 rows, in bf16 elements past a 256-byte base
OFFSET = {0: 1, 1: 4, 2: 1, 3: 8}
NAMES = ("means", "log_scales", "quats", "opacities", "sh")


def _gsr():
    import gaussian_splatting_differentiable_amd as gsr
    gsr.lib()
    return gsr


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_dev(bits, degree):
    off = OFFSET[degree]
    buf = torch.zeros(bits.size + off, dtype=torch.int16, device="cuda")
    buf[off:] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).ravel()).cuda()
    t = buf[off:].view(torch.bfloat16).view(bits.shape)
    assert t.data_ptr() % (2 * off) == 0
    return t


def rotated_scene(degree, seed, n=3000):
    rng = np.random.default_rng(seed)
    ang = rng.normal(0, 0.2, 3)
    q = np.array([1.0, *ang])
    q /= np.linalg.norm(q)
    w, x, y, z = q
    R = np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                  [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                  [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])
    t = rng.normal(0, 0.3, 3)
    cam = scenegen.pinhole(131, 77, 110.0, np.concatenate([R, t[:, None]], 1))
    pc = np.stack([rng.uniform(-1, 1, n), rng.uniform(-0.7, 0.7, n), rng.uniform(0.1, 6.0, n)], 1)
    means = ((pc - t) @ R).astype(np.float32)
    ls = rng.normal(-2.5, 0.7, (n, 3)).astype(np.float32)
    qs = rng.normal(0, 1, (n, 4)).astype(np.float32)
    op = (1 / (1 + np.exp(-rng.normal(0, 2, n)))).astype(np.float32)
    sh = rng.normal(0, 0.3, (n, (degree + 1) ** 2, 3)).astype(np.float32)
    return cam, [means, ls, qs, op, sh]


def _both_paths(gsr, cam, arrs, degree, seed):
    """fp32 calls on the widened SH and bf16 calls on the bits; host arrays."""
    means, ls, qs, op, sh = arrs
    bits, wide = scenegen.to_bf16(sh)
    n = means.shape[0]
    rng = np.random.default_rng(seed)
    g = rng.normal(0, 1, (n, 9)).astype(np.float32)
    g[rng.random(n) < 0.3] = 0.0
    r = gsr.Rasterizer(cam, capacity=16)
    d = [dev(a) for a in (means, ls, qs, op)]
    sh32, sh16 = dev(wide), bf16_dev(bits, degree)
    sp32 = host(r.project(*d, sh32, degree)).copy()
    sp16 = host(r.project(*d, sh16, degree)).copy()
    gd = dev(g)
    o32 = {k: host(v) for k, v in r.project_bwd(*d, sh32, degree, dL_dsplat=gd).items()}
    o16 = {k: host(v) for k, v in r.project_bwd(*d, sh16, degree, dL_dsplat=gd).items()}
    return wide, g, sp32, sp16, o32, o16


def _assert_bitwise(sp32, sp16, o32, o16):
    assert np.array_equal(sp32.view(np.uint32), sp16.view(np.uint32))
    for k in NAMES:
        assert np.array_equal(o32[k].view(np.uint32), o16[k].view(np.uint32)), k


@pytest.mark.parametrize("degree", [0, 1, 2, 3])
def test_bf16_calls_equal_fp32_calls_on_widened_sh(degree):
    gsr = _gsr()
    cam, arrs = rotated_scene(degree, 60 + degree)
    wide, g, sp32, sp16, o32, o16 = _both_paths(gsr, cam, arrs, degree, 70 + degree)
    _assert_bitwise(sp32, sp16, o32, o16)
    # and both against the oracle on the bf16-rounded coefficients
    means, ls, qs, op, _ = arrs
    rsp = oracle.project(means, ls, qs, op, wide, degree, cam)
    check_projection(None, rsp, sp16)
    ref = oracle.project_bwd(means, ls, qs, op, wide, degree, cam, g)
    ref["touched"] = np.any(g != 0, axis=1)
    _check(sp16, rsp, o16, ref)


@pytest.mark.parametrize("cfg", [1, 2])
def test_bf16_configs_against_oracle(cfg):
    gsr = _gsr()
    sc = scenegen.make_config(cfg)
    arrs = [sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh]
    wide, g, sp32, sp16, o32, o16 = _both_paths(gsr, sc.camera, arrs, sc.sh_degree, 80 + cfg)
    _assert_bitwise(sp32, sp16, o32, o16)
    rsp = oracle.project(sc.means, sc.log_scales, sc.quats, sc.opacities, wide, sc.sh_degree,
                         sc.camera)
    check_projection(sc, rsp, sp16)
    ref = oracle.project_bwd(sc.means, sc.log_scales, sc.quats, sc.opacities, wide, sc.sh_degree,
                             sc.camera, g)
    ref["touched"] = np.any(g != 0, axis=1)
    _check(sp16, rsp, o16, ref)


def test_bf16_garden_full_size_bitwise():
    gsr = _gsr()
    sc = scenegen.make_config(3)
    arrs = [sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh]
    _, _, sp32, sp16, o32, o16 = _both_paths(gsr, sc.camera, arrs, sc.sh_degree, 90)
    _assert_bitwise(sp32, sp16, o32, o16)
    print(f"garden bf16 SH: {int((sp16[:, 9] > 0).sum())} visible of {len(sp16)}", flush=True)
