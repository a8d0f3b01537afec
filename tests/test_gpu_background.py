"""Background colour and dL/dT_final (gs_render_fwd_bg, gs_render_bwd_bg)
against the oracle, through the C ABI.

C = sum_i c_i alpha_i T_i + T_final bg; the backward of
L = sum g . C + sum dL/dT_final T_final. Not on the pages (they blend onto
black); the plain completion of Eq. 3 of "Mitigating SM-Level Load Imbalance
in 3D Gaussian Splatting on GPUs". The bars are those of the plain stages:
rgb and T within 1e-5, gradients within 1e-3 relative L2 per column; plain
tiles and depth-chunked tiles (whose backward starts from the later chunks'
colour plus the background term) both covered.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import scenegen
from test_gpu_parity import (_gsr, check_backward, check_forward, dev, host, reference,
                             run_stages)

pytestmark = pytest.mark.gpu


def _terms(sc, seed):
    rng = np.random.default_rng(seed)
    bg = rng.uniform(-0.5, 1.0, 3).astype(np.float32)
    dT = rng.standard_normal((sc.camera.height, sc.camera.width)).astype(np.float32)
    return bg, dT


@pytest.mark.parametrize("cfg", [1, 2])
def test_background_and_dT_configs(cfg):
    gsr = _gsr()
    sc = scenegen.make_config(cfg)
    bg, dT = _terms(sc, 200 + cfg)
    ref = oracle.frame(sc, bg=bg, dL_dT=dT)
    out = run_stages(gsr, sc, ref, background=bg, dL_dT=dT)
    check_forward(ref, out)
    check_backward(ref, out)
    # the terms matter: the plain gradients would miss the 1e-3 bar by at least 2x
    plain = reference(cfg)[1]["grads"]
    assert np.linalg.norm(plain - ref["grads"]) > 2e-3 * np.linalg.norm(ref["grads"])


@pytest.mark.parametrize("bg_only", [True, False])
def test_background_ragged_scene(bg_only):
    gsr = _gsr()
    sc = scenegen.random_scene(105, 2500, 83, 45, 75.0, degree=2, log_scale=(-2.0, 0.6),
                               opacity=(1.0, 2.0))
    bg, dT = _terms(sc, 210)
    dT = None if bg_only else dT
    ref = oracle.frame(sc, bg=bg, dL_dT=dT)
    out = run_stages(gsr, sc, ref, background=bg, dL_dT=dT)
    check_forward(ref, out)
    check_backward(ref, out)


def test_dT_only_on_black():
    gsr = _gsr()
    sc = scenegen.make_config(2)
    _, dT = _terms(sc, 220)
    ref = oracle.frame(sc, dL_dT=dT)
    out = run_stages(gsr, sc, ref, background=None, dL_dT=dT)
    check_forward(ref, out)
    check_backward(ref, out)


@pytest.mark.parametrize("k,h", [(2, 0), (4, 0), (16, 40)])
def test_background_with_depth_chunks(k, h):
    gsr = _gsr()
    sc = scenegen.make_config(2) if h == 0 else scenegen.random_scene(
        104, 6000, 150, 70, 120.0, degree=1, log_scale=(-2.2, 0.7), opacity=(1.0, 2.0))
    bg, dT = _terms(sc, 230 + k)
    ref = oracle.frame(sc, bg=bg, dL_dT=dT)
    sched = gsr.make_sched(chunk_mode=2, force_k=k, force_h=h)
    out = run_stages(gsr, sc, ref, sched=sched, background=bg, dL_dT=dT)
    check_forward(ref, out)
    check_backward(ref, out)
    assert out["plan"]["k"] == k


def test_black_background_calls_equal_plain_calls():
    """A zero background through the _bg entry points takes the plain path: the
    forward is bit for bit the plain call's; the backward (whose float atomics
    may add in another order) meets the usual bar."""
    gsr = _gsr()
    sc, ref = reference(2)
    a = run_stages(gsr, sc, ref)
    b = run_stages(gsr, sc, ref, background=np.zeros(3, np.float32))
    assert np.array_equal(a["rgb"].view(np.uint32), b["rgb"].view(np.uint32))
    assert np.array_equal(a["T"].view(np.uint32), b["T"].view(np.uint32))
    check_backward(ref, b)


def test_background_rejects_non_finite():
    gsr = _gsr()
    sc, ref = reference(1)
    with pytest.raises(gsr.GsError):
        run_stages(gsr, sc, ref, background=np.array([np.nan, 0, 0], np.float32))


def test_background_garden_full_size():
    gsr = _gsr()
    sc = scenegen.make_config(3)
    bg, dT = _terms(sc, 240)
    ref = oracle.frame(sc, bg=bg, dL_dT=dT)
    out = run_stages(gsr, sc, ref, background=bg, dL_dT=dT)
    check_forward(ref, out)
    check_backward(ref, out)
