"""The HIP library loads on the CPU host and exports every function that
include/gs.h declares; host-only functions and argument validation work
without touching a GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gs.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def gsr():
    import gaussian_splatting_differentiable_amd as g
    if not os.path.exists(g.LIB_PATH):
        pytest.skip("libgs.so not built (run __graft_entry__.build())")
    g.lib()
    return g


def test_every_declared_symbol_is_exported(gsr):
    names = _declared()
    assert set(names) == set(gsr.EXPORTS), names
    L = C.CDLL(gsr.LIB_PATH)
    for name in names:
        assert hasattr(L, name), name


def test_strerror_and_sizes(gsr):
    assert gsr.strerror(0) == "ok"
    assert "capacity" in gsr.strerror(gsr.GS_ERR_CAPACITY)
    assert "wait" in gsr.strerror(gsr.GS_ERR_TIMEOUT)
    ws = gsr.workspace_size(1_535_033, 1297, 840, 8_000_000)
    assert ws > 8_000_000 * 16
    assert gsr.workspace_size(-1, 10, 10, 0) == 0
    # the forward state grows by the contributor record: 4 bits per pair
    a, b = gsr.fwd_state_size(1297, 840, 0), gsr.fwd_state_size(1297, 840, 8_000_000)
    assert a >= 4346 * 4 * 4 and 8_000_000 // 2 <= b - a <= 8_000_000 // 2 + 32 * 4346 + 512
    assert gsr.fwd_state_size(0, 10, 100) == 0
    assert gsr.fwd_state_size(10, 10, -1) == 0 and gsr.fwd_state_size(10, 10, 1 << 30) == 0


def test_argument_validation_needs_no_gpu(gsr):
    L = gsr.lib()
    cam = gsr.GsCamera()
    cam.width, cam.height, cam.fx, cam.fy = 64, 64, 64.0, 64.0
    # negative n, bad degree and a bad camera are rejected before any HIP call
    assert L.gs_project(-1, None, None, None, None, None, 0, C.byref(cam), None, None) == -1
    assert L.gs_project(4, None, None, None, None, None, 7, C.byref(cam), None, None) == -1
    bad = gsr.GsCamera()
    assert L.gs_project(1, None, None, None, None, None, 0, C.byref(bad), None, None) == -1
    # the projection backward: the same checks, plus missing outputs and misaligned quaternions
    nul = [None] * 6
    assert L.gs_project_bwd(-1, None, None, None, None, None, 0, C.byref(cam), *nul, None) == -1
    assert L.gs_project_bwd(4, None, None, None, None, None, 4, C.byref(cam), *nul, None) == -1
    assert L.gs_project_bwd(1, None, None, None, None, None, 0, C.byref(bad), *nul, None) == -1
    p16 = C.c_void_p(16)
    assert L.gs_project_bwd(1, p16, p16, p16, p16, p16, 0, C.byref(cam), p16, p16, p16, p16, p16,
                            None, None) == -1
    assert L.gs_project_bwd(1, p16, p16, C.c_void_p(20), p16, p16, 0, C.byref(cam), p16, p16, p16,
                            p16, p16, p16, None) == -1
    assert L.gs_project_bwd(0, None, None, None, None, None, 0, C.byref(cam), *nul, None) == 0
    # bf16 SH: rows of degree 3 need 16-byte, of degree 1 8-byte, else 2-byte alignment
    for deg, addr in ((3, 24), (1, 20), (0, 17), (2, 33)):
        sh = C.c_void_p(addr)
        assert L.gs_project_bf16sh(1, p16, p16, p16, p16, sh, deg, C.byref(cam), p16, None) == -1
        assert L.gs_project_bwd_bf16sh(1, p16, p16, p16, p16, sh, deg, C.byref(cam), p16, p16,
                                       p16, p16, p16, p16, None) == -1
    # the SH gradient stays fp32: 16-byte aligned rows for degrees 1 and 3
    assert L.gs_project_bwd_bf16sh(1, p16, p16, p16, p16, p16, 3, C.byref(cam), p16, p16, p16,
                                   p16, p16, C.c_void_p(24), None) == -1
    assert L.gs_project_bf16sh(-1, None, None, None, None, None, 0, C.byref(cam), None, None) == -1
    assert L.gs_project_bwd_bf16sh(0, None, None, None, None, None, 0, C.byref(cam), *nul,
                                   None) == 0
    # background: non-finite values and a misaligned dL/dT_final are rejected before any HIP call
    nanbg = (C.c_float * 3)(float("nan"), 0.0, 0.0)
    st256 = C.c_void_p(256)
    assert L.gs_render_fwd_bg(1, p16, p16, p16, C.byref(cam), None, p16, p16, p16, st256, 1 << 30,
                              None, None, p16, nanbg, None) == -1
    assert L.gs_render_bwd_bg(1, p16, p16, p16, C.byref(cam), p16, p16, st256, 1 << 30, p16, p16,
                              p16, nanbg, None, None) == -1
    assert L.gs_render_bwd_bg(1, p16, p16, p16, C.byref(cam), p16, p16, st256, 1 << 30, p16, p16,
                              p16, None, C.c_void_p(18), None) == -1
    # the frame's device status word is required by the sort and the raster calls
    assert L.gs_render_fwd(1, p16, p16, p16, C.byref(cam), None, p16, p16, p16, st256, 1 << 30,
                           None, None, None, None) == -1
    assert L.gs_render_bwd(1, p16, p16, p16, C.byref(cam), p16, p16, st256, 1 << 30, p16, p16,
                           None, None) == -1
    assert L.gs_sort_keys(10, p16, p16, 100, C.byref(cam), None, p16, p16, None, p16, 1 << 30,
                          None) == -1
    # a forward state too small for even an empty contributor record
    small = L.gs_fwd_state_size(64, 64, 0) - 256
    assert L.gs_render_fwd(1, p16, p16, p16, C.byref(cam), None, p16, p16, p16, st256, small,
                           None, None, p16, None) == -3
    assert L.gs_render_bwd(1, p16, p16, p16, C.byref(cam), p16, p16, st256, small, p16, p16,
                           p16, None) == -3
    # counts from 2^30 up: the radix passes' look-back words hold 30-bit counts
    big_ws = C.c_size_t(1 << 62)
    assert L.gs_bin_tiles(1 << 30, p16, C.byref(cam), 100, p16, None, None, None, p16, p16,
                          big_ws, None) == -5
    assert L.gs_bin_tiles(10, p16, C.byref(cam), 1 << 30, p16, None, None, None, p16, p16,
                          big_ws, None) == -5
    assert L.gs_sort_keys(10, p16, p16, 1 << 30, C.byref(cam), None, p16, p16, p16, p16, big_ws,
                          None) == -5
    assert L.gs_render_fwd(1 << 30, p16, p16, p16, C.byref(cam), None, p16, p16, p16, st256,
                           1 << 40, None, None, p16, None) == -5
    # batches of views: sizes are those of the stacked image; bad batches are rejected
    assert L.gs_fwd_state_size_views(64, 45, 3, 500) == L.gs_fwd_state_size(64, 3 * 48, 500)
    assert L.gs_workspace_size_views(1000, 83, 45, 4, 5000) == L.gs_workspace_size(1000, 83, 4 * 48,
                                                                                    5000)
    assert L.gs_fwd_state_size_views(64, 64, 0, 8) == 0
    assert L.gs_fwd_state_size_views(64, 64, 17, 8) == 0
    assert L.gs_bin_tiles_views(1, p16, C.byref(cam), 0, 10, p16, None, None, None, p16, p16,
                                1 << 30, None) == -1
    assert L.gs_render_fwd_views(1, p16, p16, p16, C.byref(cam), 17, None, p16, p16, p16, st256,
                                 1 << 30, None, None, p16, None, None) == -1
    assert L.gs_project_views(1, p16, p16, p16, p16, p16, 0, None, 2, p16, None) == -1
    cams2 = (gsr.GsCamera * 2)(cam, cam)
    cams2[1].width = 80                                   # views of different sizes
    assert L.gs_project_views(1, p16, p16, p16, p16, p16, 0, cams2, 2, p16, None) == -1
    assert L.gs_project_bwd_views(1, p16, p16, p16, p16, p16, 0, cams2, 2, p16, p16, p16, p16, p16,
                                  p16, None) == -1
    big = gsr.GsCamera()
    big.width, big.height, big.fx, big.fy = 1 << 14, 1 << 14, 1.0, 1.0
    assert L.gs_bin_tiles(1, C.c_void_p(16), C.byref(big), 10, C.c_void_p(16), None,
                          C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), 1 << 30,
                          None) == -5
    # undersized workspace
    assert L.gs_bin_tiles(10, C.c_void_p(16), C.byref(cam), 100, C.c_void_p(16), None,
                          C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), 8,
                          None) == -3
    # the wait limit is host state: set, read back, restored
    prev = L.gs_set_wait_limit(5)
    assert prev == -1
    assert L.gs_set_wait_limit(-3) == 5
    assert L.gs_set_wait_limit(-1) == -1
    # a misaligned tile-count array
    assert L.gs_bin_tiles(10, p16, C.byref(cam), 100, p16, C.c_void_p(18), None, None, p16, p16,
                          1 << 30, None) == -1
    # the plan built ahead: counts, state and status are required; the state must
    # hold the header and arrays; knobs are checked as for the forward
    assert L.gs_plan_tiles(None, C.byref(cam), None, st256, 1 << 30, p16, None) == -1
    assert L.gs_plan_tiles(p16, C.byref(cam), None, None, 1 << 30, p16, None) == -1
    assert L.gs_plan_tiles(p16, C.byref(cam), None, st256, 1 << 30, None, None) == -1
    assert L.gs_plan_tiles(C.c_void_p(18), C.byref(cam), None, st256, 1 << 30, p16, None) == -1
    assert L.gs_plan_tiles(p16, C.byref(cam), None, C.c_void_p(272), 1 << 30, p16, None) == -1
    assert L.gs_plan_tiles(p16, C.byref(cam), None, st256, small, p16, None) == -3
    bad_sched = gsr.make_sched(chunk_mode=3)
    assert L.gs_plan_tiles(p16, C.byref(cam), C.byref(bad_sched), st256, 1 << 30, p16,
                           None) == -1
    assert L.gs_plan_tiles(p16, C.byref(bad), None, st256, 1 << 30, p16, None) == -1
    assert L.gs_plan_tiles_views(p16, C.byref(cam), 17, None, st256, 1 << 30, p16, None) == -1
    assert L.gs_plan_tiles(p16, C.byref(big), None, st256, 1 << 40, p16, None) == -5


def test_forward_clear_argument_validation_needs_no_gpu(gsr):
    """gs_render_fwd_zero: a negative count, a missing or misaligned array with a
    positive count are rejected before any HIP call."""
    L = gsr.lib()
    cam = gsr.GsCamera()
    cam.width, cam.height, cam.fx, cam.fy = 64, 64, 64.0, 64.0
    p16 = C.c_void_p(1 << 20)
    st256 = gsr.fwd_state_size(64, 64, 1 << 10)
    common = (1, p16, p16, p16, C.byref(cam), None, p16, p16, p16, p16, st256, None, None, p16,
              None)
    assert L.gs_render_fwd_zero(*common, p16, -1, None) == gsr.GS_ERR_INVALID_ARGUMENT
    assert L.gs_render_fwd_zero(*common, None, 16, None) == gsr.GS_ERR_INVALID_ARGUMENT
    assert L.gs_render_fwd_zero(*common, C.c_void_p((1 << 20) + 4), 16,
                                None) == gsr.GS_ERR_INVALID_ARGUMENT


def test_sort_with_plan_argument_validation_needs_no_gpu(gsr):
    """gs_sort_keys_plan: a missing or misaligned forward state, one too small for
    the tile grid, and bad schedule knobs are rejected before any HIP call."""
    L = gsr.lib()
    cam = gsr.GsCamera()
    cam.width, cam.height, cam.fx, cam.fy = 64, 64, 64.0, 64.0
    p = C.c_void_p(1 << 20)
    st = gsr.fwd_state_size(64, 64, 1 << 10)
    ws = gsr.workspace_size(16, 64, 64, 1 << 10)
    args = lambda sched, fs, fsb: (16, p, p, 1 << 10, C.byref(cam), None, p, p, sched, fs, fsb, p, p,
                                   ws, None)
    assert L.gs_sort_keys_plan(*args(None, None, st)) == gsr.GS_ERR_INVALID_ARGUMENT
    assert L.gs_sort_keys_plan(*args(None, C.c_void_p((1 << 20) + 64), st)) == \
        gsr.GS_ERR_INVALID_ARGUMENT
    assert L.gs_sort_keys_plan(*args(None, p, 64)) == gsr.GS_ERR_WORKSPACE
    bad = gsr.make_sched(chunk_mode=3)
    assert L.gs_sort_keys_plan(*args(C.byref(bad), p, st)) == gsr.GS_ERR_INVALID_ARGUMENT
    # the forward refuses a `planned` value other than 0 and 1
    odd = gsr.make_sched(planned=2)
    assert L.gs_render_fwd(1, p, p, p, C.byref(cam), C.byref(odd), p, p, p, p, st, None, None, p,
                           None) == gsr.GS_ERR_INVALID_ARGUMENT
