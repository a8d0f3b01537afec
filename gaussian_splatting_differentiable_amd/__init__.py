"""MI355X-native tile-based differentiable Gaussian-splatting rasterizer.

The work runs in hand-written HIP kernels behind the C ABI declared in
``include/gs.h`` (``libgs.so`` in this package directory). This module is the
thin Python binding: it marshals torch tensors (device memory) and the current
HIP stream into those calls and raises ``GsError`` on a bad status. It does no
arithmetic of its own, and it fails loudly when the library has not been built.

Low-level calls keep the C names (``gs_project``, ``gs_bin_tiles``,
``gs_sort_keys``, ``gs_render_fwd``, ``gs_render_bwd``); ``Rasterizer`` owns the
scratch buffers and chains them into a frame.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgs.so")

GS_OK, GS_ERR_INVALID_ARGUMENT, GS_ERR_CAPACITY = 0, -1, -2
GS_ERR_WORKSPACE, GS_ERR_HIP, GS_ERR_UNSUPPORTED, GS_ERR_TIMEOUT = -3, -4, -5, -6
SPLAT_FLOATS, GRAD_FLOATS, TILE = 12, 9, 16

EXPORTS = ("gs_strerror", "gs_workspace_size", "gs_fwd_state_size", "gs_project", "gs_project_bwd",
           "gs_project_bf16sh", "gs_project_bwd_bf16sh", "gs_bin_tiles",
           "gs_render_fwd_bg", "gs_render_bwd_bg", "gs_workspace_size_views",
           "gs_fwd_state_size_views", "gs_project_views", "gs_project_bwd_views",
           "gs_bin_tiles_views", "gs_sort_keys_views", "gs_render_fwd_views",
           "gs_render_bwd_views", "gs_sort_keys", "gs_render_fwd", "gs_render_bwd",
           "gs_sort_keys_noalloc", "gs_plan_tiles", "gs_plan_tiles_views", "gs_timing_start",
           "gs_timing_read", "gs_set_wait_limit", "gs_render_bwd_accumulate",
           "gs_render_fwd_zero", "gs_sort_keys_plan")
NOALLOC_SCRATCH_BYTES = 64 << 20


class GsError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} ({status})")


class GsCamera(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("world_to_cam", C.c_float * 12),
                ("znear", C.c_float), ("lowpass", C.c_float)]


class GsSched(C.Structure):
    _fields_ = [("chunk_mode", C.c_int32), ("force_k", C.c_int32), ("force_h", C.c_int32),
                ("lambda_", C.c_float), ("beta", C.c_float), ("eps", C.c_float),
                ("planned", C.c_int32)]


_lib_handle = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = C.CDLL(LIB_PATH)
    P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    cam_p = C.POINTER(GsCamera)
    L.gs_strerror.argtypes, L.gs_strerror.restype = [i32], C.c_char_p
    L.gs_workspace_size.argtypes, L.gs_workspace_size.restype = [i32, i32, i32, i64], sz
    L.gs_fwd_state_size.argtypes, L.gs_fwd_state_size.restype = [i32, i32, i64], sz
    L.gs_project.argtypes = [i32, P, P, P, P, P, i32, cam_p, P, P]
    L.gs_project_bwd.argtypes = [i32, P, P, P, P, P, i32, cam_p, P, P, P, P, P, P, P]
    L.gs_project_bf16sh.argtypes = L.gs_project.argtypes
    L.gs_project_bwd_bf16sh.argtypes = L.gs_project_bwd.argtypes
    L.gs_bin_tiles.argtypes = [i32, P, cam_p, i64, P, P, P, P, P, P, sz, P]
    L.gs_sort_keys.argtypes = [i32, P, P, i64, cam_p, P, P, P, P, P, sz, P]
    L.gs_render_fwd.argtypes = [i32, P, P, P, cam_p, C.POINTER(GsSched), P, P, P, P, sz, P, P, P,
                                P]
    L.gs_render_bwd.argtypes = [i32, P, P, P, cam_p, P, P, P, sz, P, P, P, P]
    L.gs_render_fwd_bg.argtypes = L.gs_render_fwd.argtypes[:-1] + [P, P]
    L.gs_render_bwd_bg.argtypes = L.gs_render_bwd.argtypes[:-1] + [P, P, P]
    L.gs_render_fwd_zero.argtypes = L.gs_render_fwd.argtypes[:-1] + [P, P, i64, P]
    L.gs_sort_keys_plan.argtypes = [i32, P, P, i64, cam_p, P, P, P, C.POINTER(GsSched), P, sz, P,
                                    P, sz, P]
    L.gs_workspace_size_views.argtypes = [i32, i32, i32, i32, i64]
    L.gs_workspace_size_views.restype = sz
    L.gs_fwd_state_size_views.argtypes = [i32, i32, i32, i64]
    L.gs_fwd_state_size_views.restype = sz
    L.gs_project_views.argtypes = [i32, P, P, P, P, P, i32, cam_p, i32, P, P]
    L.gs_project_bwd_views.argtypes = [i32, P, P, P, P, P, i32, cam_p, i32, P, P, P, P, P, P, P]
    L.gs_bin_tiles_views.argtypes = [i32, P, cam_p, i32, i64, P, P, P, P, P, P, sz, P]
    L.gs_plan_tiles.argtypes = [P, cam_p, C.POINTER(GsSched), P, sz, P, P]
    L.gs_plan_tiles_views.argtypes = [P, cam_p, i32, C.POINTER(GsSched), P, sz, P, P]
    L.gs_sort_keys_views.argtypes = [i32, P, P, i64, cam_p, i32, P, P, P, P, P, sz, P]
    L.gs_render_fwd_views.argtypes = [i32, P, P, P, cam_p, i32, C.POINTER(GsSched), P, P, P, P,
                                      sz, P, P, P, P, P]
    L.gs_render_bwd_views.argtypes = [i32, P, P, P, cam_p, i32, P, P, P, sz, P, P, P, P, P, P]
    L.gs_render_bwd_accumulate.argtypes = [i32, P, P, P, cam_p, i32, P, P, P, sz, P, P, P, P, P,
                                           P]
    L.gs_sort_keys_noalloc.argtypes = [i32, P, cam_p, i64, P, P, P, P, P, P]
    L.gs_timing_start.argtypes = []
    L.gs_set_wait_limit.argtypes = [i32]
    L.gs_timing_read.argtypes = [i32, C.POINTER(C.c_float), i32]
    for name in ("gs_project", "gs_project_bwd", "gs_project_bf16sh", "gs_project_bwd_bf16sh",
                 "gs_bin_tiles", "gs_render_fwd_bg", "gs_render_bwd_bg", "gs_project_views",
                 "gs_project_bwd_views", "gs_bin_tiles_views", "gs_sort_keys_views",
                 "gs_render_fwd_views", "gs_render_bwd_views", "gs_sort_keys", "gs_render_fwd",
                 "gs_render_bwd", "gs_sort_keys_noalloc", "gs_plan_tiles", "gs_plan_tiles_views",
                 "gs_timing_start", "gs_timing_read", "gs_set_wait_limit",
                 "gs_render_bwd_accumulate", "gs_render_fwd_zero", "gs_sort_keys_plan"):
        getattr(L, name).restype = i32
    _lib_handle = L
    return L


def strerror(status: int) -> str:
    return lib().gs_strerror(int(status)).decode()


def make_camera(cam) -> GsCamera:
    """GsCamera from any object with width, height, fx, fy, cx, cy, world_to_cam, znear, lowpass."""
    c = GsCamera()
    c.width, c.height = int(cam.width), int(cam.height)
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    for i, v in enumerate(list(cam.world_to_cam)):
        c.world_to_cam[i] = float(v)
    c.znear, c.lowpass = float(cam.znear), float(cam.lowpass)
    return c


# Defaults of the per-frame chunking policy (Eq. 6 constants; the page does not
# print lambda and beta, these are calibrated for this build).
DEFAULT_LAMBDA, DEFAULT_BETA, DEFAULT_EPS = 131072.0, 0.25, 0.10
HK_MAX = 4096  # cap on h*k, the chunks of chunked tiles per frame


def make_sched(chunk_mode: int = 1, force_k: int = 0, force_h: int = 0,
               lambda_: float = DEFAULT_LAMBDA, beta: float = DEFAULT_BETA,
               eps: float = DEFAULT_EPS, planned: int = 0) -> GsSched:
    return GsSched(int(chunk_mode), int(force_k), int(force_h), float(lambda_), float(beta),
                   float(eps), int(planned))


TILE_PASS_PARTITION = 16384  # pairs per partition of the sort's tile passes


def plan_in_sort(tiles: int, pairs: int) -> bool:
    """Whether gs_sort_keys_plan hides the tile schedule (about 30 us in one
    workgroup) inside the sort: the frame has a 5-bit tile pass (257 to 8192
    tiles) with at least one round of partitions on every compute unit. Other
    frames build the schedule beside the sort on a second stream."""
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    return 256 < tiles <= 8192 and pairs >= cus * TILE_PASS_PARTITION


def planned_sched(sched) -> GsSched:
    """A copy of sched (None: the defaults) for a forward whose plan was built
    ahead with gs_plan_tiles on a stream it waits for."""
    s = make_sched() if sched is None else GsSched.from_buffer_copy(sched)
    s.planned = 1
    return s


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _check(status, what):
    if status != GS_OK:
        raise GsError(status, what)


def workspace_size(n, width, height, capacity) -> int:
    return int(lib().gs_workspace_size(int(n), int(width), int(height), int(capacity)))


def fwd_state_size(width, height, capacity) -> int:
    return int(lib().gs_fwd_state_size(int(width), int(height), int(capacity)))


def workspace_size_views(n, width, height, n_views, capacity) -> int:
    return int(lib().gs_workspace_size_views(int(n), int(width), int(height), int(n_views),
                                             int(capacity)))


def fwd_state_size_views(width, height, n_views, capacity) -> int:
    return int(lib().gs_fwd_state_size_views(int(width), int(height), int(n_views),
                                             int(capacity)))


def _cams(cams):
    """A C array of cameras from scenegen cameras or GsCamera values."""
    arr = (GsCamera * len(cams))()
    for i, c in enumerate(cams):
        arr[i] = c if isinstance(c, GsCamera) else make_camera(c)
    return arr


def gs_project_views(n, means, log_scales, quats, opacities, sh, sh_degree, cams, splats,
                     stream=None):
    arr = _cams(cams)
    _check(lib().gs_project_views(int(n), _ptr(means), _ptr(log_scales), _ptr(quats),
                                  _ptr(opacities), _ptr(sh), int(sh_degree), arr, len(cams),
                                  _ptr(splats), _stream(stream)),
           "gs_project_views")


def gs_project_bwd_views(n, means, log_scales, quats, opacities, sh, sh_degree, cams, dL_dsplat,
                         dL_dmeans, dL_dlog_scales, dL_dquats, dL_dopacities, dL_dsh,
                         stream=None):
    arr = _cams(cams)
    _check(lib().gs_project_bwd_views(int(n), _ptr(means), _ptr(log_scales), _ptr(quats),
                                      _ptr(opacities), _ptr(sh), int(sh_degree), arr, len(cams),
                                      _ptr(dL_dsplat), _ptr(dL_dmeans), _ptr(dL_dlog_scales),
                                      _ptr(dL_dquats), _ptr(dL_dopacities), _ptr(dL_dsh),
                                      _stream(stream)),
           "gs_project_bwd_views")


def gs_bin_tiles_views(n, splats, cam, n_views, capacity, offsets, keys, ids, status, workspace,
                       stream=None, tile_counts=None):
    _check(lib().gs_bin_tiles_views(int(n), _ptr(splats), C.byref(cam), int(n_views),
                                    int(capacity), _ptr(offsets), _ptr(tile_counts), _ptr(keys),
                                    _ptr(ids),
                                    _ptr(status), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(stream)),
           "gs_bin_tiles_views")


def gs_sort_keys_views(n, splats, offsets, capacity, cam, n_views, sorted_keys, sorted_ids,
                       ranges, status, workspace, stream=None):
    _check(lib().gs_sort_keys_views(int(n), _ptr(splats), _ptr(offsets), int(capacity),
                                    C.byref(cam), int(n_views), _ptr(sorted_keys),
                                    _ptr(sorted_ids), _ptr(ranges), _ptr(status),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)),
           "gs_sort_keys_views")


def gs_render_fwd_views(n, splats, sorted_ids, ranges, cam, n_views, sched, rgb, T_final, last,
                        fwd_state, stats, pixel_hits, status, background=None, stream=None):
    _check(lib().gs_render_fwd_views(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges),
                                     C.byref(cam), int(n_views),
                                     C.byref(sched) if sched is not None else None, _ptr(rgb),
                                     _ptr(T_final), _ptr(last), _ptr(fwd_state),
                                     fwd_state.numel() * fwd_state.element_size(), _ptr(stats),
                                     _ptr(pixel_hits), _ptr(status), _bg3(background),
                                     _stream(stream)),
           "gs_render_fwd_views")


def gs_render_bwd_views(n, splats, sorted_ids, ranges, cam, n_views, T_final, last, fwd_state,
                        dL_drgb, dL_dsplat, status, background=None, dL_dT=None, stream=None):
    _check(lib().gs_render_bwd_views(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges),
                                     C.byref(cam), int(n_views), _ptr(T_final), _ptr(last),
                                     _ptr(fwd_state), fwd_state.numel() * fwd_state.element_size(),
                                     _ptr(dL_drgb), _ptr(dL_dsplat), _ptr(status),
                                     _bg3(background), _ptr(dL_dT), _stream(stream)),
           "gs_render_bwd_views")


def gs_render_fwd_zero(n, splats, sorted_ids, ranges, cam, sched, rgb, T_final, last, fwd_state,
                       stats, pixel_hits, status, zero_out, background=None, stream=None):
    """gs_render_fwd_bg that also clears zero_out (every element), e.g. the
    gradient array a gs_render_bwd_accumulate of the frame adds into."""
    _check(lib().gs_render_fwd_zero(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges),
                                    C.byref(cam), C.byref(sched) if sched is not None else None,
                                    _ptr(rgb), _ptr(T_final), _ptr(last), _ptr(fwd_state),
                                    fwd_state.numel() * fwd_state.element_size(), _ptr(stats),
                                    _ptr(pixel_hits), _ptr(status), _bg3(background),
                                    _ptr(zero_out), int(zero_out.numel()), _stream(stream)),
           "gs_render_fwd_zero")


def gs_render_bwd_accumulate(n, splats, sorted_ids, ranges, cam, n_views, T_final, last,
                             fwd_state, dL_drgb, dL_dsplat, status, background=None, dL_dT=None,
                             stream=None):
    """gs_render_bwd_views (any n_views >= 1) adding into dL_dsplat, which the
    caller initialises."""
    _check(lib().gs_render_bwd_accumulate(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges),
                                          C.byref(cam), int(n_views), _ptr(T_final), _ptr(last),
                                          _ptr(fwd_state),
                                          fwd_state.numel() * fwd_state.element_size(),
                                          _ptr(dL_drgb), _ptr(dL_dsplat), _ptr(status),
                                          _bg3(background), _ptr(dL_dT), _stream(stream)),
           "gs_render_bwd_accumulate")


# ------------------------------------------------------------------ C-named calls

def gs_project(n, means, log_scales, quats, opacities, sh, sh_degree, cam, splats, stream=None):
    _check(lib().gs_project(int(n), _ptr(means), _ptr(log_scales), _ptr(quats), _ptr(opacities),
                            _ptr(sh), int(sh_degree), C.byref(cam), _ptr(splats), _stream(stream)),
           "gs_project")


def gs_project_bwd(n, means, log_scales, quats, opacities, sh, sh_degree, cam, dL_dsplat,
                   dL_dmeans, dL_dlog_scales, dL_dquats, dL_dopacities, dL_dsh, stream=None):
    _check(lib().gs_project_bwd(int(n), _ptr(means), _ptr(log_scales), _ptr(quats),
                                _ptr(opacities), _ptr(sh), int(sh_degree), C.byref(cam),
                                _ptr(dL_dsplat), _ptr(dL_dmeans), _ptr(dL_dlog_scales),
                                _ptr(dL_dquats), _ptr(dL_dopacities), _ptr(dL_dsh),
                                _stream(stream)),
           "gs_project_bwd")


def gs_project_bf16sh(n, means, log_scales, quats, opacities, sh, sh_degree, cam, splats,
                      stream=None):
    _check(lib().gs_project_bf16sh(int(n), _ptr(means), _ptr(log_scales), _ptr(quats),
                                   _ptr(opacities), _ptr(sh), int(sh_degree), C.byref(cam),
                                   _ptr(splats), _stream(stream)),
           "gs_project_bf16sh")


def gs_project_bwd_bf16sh(n, means, log_scales, quats, opacities, sh, sh_degree, cam, dL_dsplat,
                          dL_dmeans, dL_dlog_scales, dL_dquats, dL_dopacities, dL_dsh,
                          stream=None):
    _check(lib().gs_project_bwd_bf16sh(int(n), _ptr(means), _ptr(log_scales), _ptr(quats),
                                       _ptr(opacities), _ptr(sh), int(sh_degree), C.byref(cam),
                                       _ptr(dL_dsplat), _ptr(dL_dmeans), _ptr(dL_dlog_scales),
                                       _ptr(dL_dquats), _ptr(dL_dopacities), _ptr(dL_dsh),
                                       _stream(stream)),
           "gs_project_bwd_bf16sh")


def gs_bin_tiles(n, splats, cam, capacity, offsets, keys, ids, status, workspace, stream=None,
                 tile_counts=None):
    _check(lib().gs_bin_tiles(int(n), _ptr(splats), C.byref(cam), int(capacity), _ptr(offsets),
                              _ptr(tile_counts), _ptr(keys), _ptr(ids), _ptr(status),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)),
           "gs_bin_tiles")


def gs_plan_tiles(tile_counts, cam, sched, fwd_state, status, stream=None):
    _check(lib().gs_plan_tiles(_ptr(tile_counts), C.byref(cam),
                               C.byref(sched) if sched is not None else None, _ptr(fwd_state),
                               fwd_state.numel() * fwd_state.element_size(), _ptr(status),
                               _stream(stream)),
           "gs_plan_tiles")


def gs_plan_tiles_views(tile_counts, cam, n_views, sched, fwd_state, status, stream=None):
    _check(lib().gs_plan_tiles_views(_ptr(tile_counts), C.byref(cam), int(n_views),
                                     C.byref(sched) if sched is not None else None,
                                     _ptr(fwd_state), fwd_state.numel() * fwd_state.element_size(),
                                     _ptr(status), _stream(stream)),
           "gs_plan_tiles_views")


def gs_sort_keys(n, splats, offsets, capacity, cam, sorted_keys, sorted_ids, ranges, status,
                 workspace, stream=None):
    _check(lib().gs_sort_keys(int(n), _ptr(splats), _ptr(offsets), int(capacity), C.byref(cam),
                              _ptr(sorted_keys), _ptr(sorted_ids), _ptr(ranges), _ptr(status),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)),
           "gs_sort_keys")


def gs_sort_keys_plan(n, splats, offsets, capacity, cam, sorted_keys, sorted_ids, ranges, sched,
                      fwd_state, status, workspace, stream=None):
    """gs_sort_keys that also builds the frame's tile schedule into fwd_state, for
    a forward with planned_sched(sched) on the same stream."""
    _check(lib().gs_sort_keys_plan(int(n), _ptr(splats), _ptr(offsets), int(capacity),
                                   C.byref(cam), _ptr(sorted_keys), _ptr(sorted_ids), _ptr(ranges),
                                   C.byref(sched) if sched is not None else None, _ptr(fwd_state),
                                   fwd_state.numel() * fwd_state.element_size(), _ptr(status),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)),
           "gs_sort_keys_plan")


def gs_render_fwd(n, splats, sorted_ids, ranges, cam, sched, rgb, T_final, last, fwd_state,
                  stats, pixel_hits, status, stream=None):
    _check(lib().gs_render_fwd(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges), C.byref(cam),
                               C.byref(sched) if sched is not None else None, _ptr(rgb),
                               _ptr(T_final), _ptr(last), _ptr(fwd_state),
                               fwd_state.numel() * fwd_state.element_size(), _ptr(stats),
                               _ptr(pixel_hits), _ptr(status), _stream(stream)),
           "gs_render_fwd")


def gs_render_bwd(n, splats, sorted_ids, ranges, cam, T_final, last, fwd_state, dL_drgb,
                  dL_dsplat, status, stream=None):
    _check(lib().gs_render_bwd(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges), C.byref(cam),
                               _ptr(T_final), _ptr(last), _ptr(fwd_state),
                               fwd_state.numel() * fwd_state.element_size(), _ptr(dL_drgb),
                               _ptr(dL_dsplat), _ptr(status), _stream(stream)),
           "gs_render_bwd")


def gs_sort_keys_noalloc(n, splats, cam, capacity, offsets, sorted_keys, sorted_ids, ranges,
                         status, stream=None):
    _check(lib().gs_sort_keys_noalloc(int(n), _ptr(splats), C.byref(cam), int(capacity),
                                      _ptr(offsets), _ptr(sorted_keys), _ptr(sorted_ids),
                                      _ptr(ranges), _ptr(status), _stream(stream)),
           "gs_sort_keys_noalloc")


def _bg3(background):
    """A host array of 3 floats for the C call, or None (black)."""
    if background is None:
        return None
    vals = [float(v) for v in background]
    if len(vals) != 3:
        raise ValueError("background takes 3 values")
    return (C.c_float * 3)(*vals)


def gs_render_fwd_bg(n, splats, sorted_ids, ranges, cam, sched, rgb, T_final, last, fwd_state,
                     stats, pixel_hits, status, background, stream=None):
    _check(lib().gs_render_fwd_bg(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges),
                                  C.byref(cam), C.byref(sched) if sched is not None else None,
                                  _ptr(rgb), _ptr(T_final), _ptr(last), _ptr(fwd_state),
                                  fwd_state.numel() * fwd_state.element_size(), _ptr(stats),
                                  _ptr(pixel_hits), _ptr(status), _bg3(background),
                                  _stream(stream)),
           "gs_render_fwd_bg")


def gs_render_bwd_bg(n, splats, sorted_ids, ranges, cam, T_final, last, fwd_state, dL_drgb,
                     dL_dsplat, status, background, dL_dT, stream=None):
    _check(lib().gs_render_bwd_bg(int(n), _ptr(splats), _ptr(sorted_ids), _ptr(ranges),
                                  C.byref(cam), _ptr(T_final), _ptr(last), _ptr(fwd_state),
                                  fwd_state.numel() * fwd_state.element_size(), _ptr(dL_drgb),
                                  _ptr(dL_dsplat), _ptr(status), _bg3(background), _ptr(dL_dT),
                                  _stream(stream)),
           "gs_render_bwd_bg")


def gs_timing_start():
    _check(lib().gs_timing_start(), "gs_timing_start")


def gs_set_wait_limit(probes: int) -> int:
    """Probe limit of the bounded device-side waits (below 0: their defaults);
    returns the previous setting. For tests of the give-up path."""
    return int(lib().gs_set_wait_limit(int(probes)))


def gs_timing_read(which: int, cap: int = 512):
    """Durations (ms) of the raster kernel launches recorded since gs_timing_start;
    which 0 = k_render_fwd, 1 = k_render_bwd."""
    buf = (C.c_float * cap)()
    n = lib().gs_timing_read(int(which), buf, int(cap))
    if n < 0:
        raise GsError(n, "gs_timing_read")
    return [float(buf[i]) for i in range(n)]


# ------------------------------------------------------------------ frame driver

class Rasterizer:
    """Owns the per-frame buffers for one image size and chains the five calls.

    Every call only enqueues work on the current stream. The frame's device
    status word is read once, after the frame (``frame_status``); ``run_frame``
    chains a whole frame and, when the pairs overflowed the buffers, grows them
    and runs the frame again. With plan_ahead the tile schedule is built
    before the forward needs it: for one view inside the sort
    (gs_sort_keys_plan), for a batch of views from the binning pass's tile
    counts on a second stream while the sort runs (gs_plan_tiles_views); the
    forward then checks it in its own launch (sched.planned).
    """

    def __init__(self, camera, device="cuda", capacity=1 << 20, sched=None, n_views=1,
                 plan_ahead=True):
        """n_views > 1: a batch of views of camera's size (the *_views calls); the
        outputs stack the views' rows and `n` counts splat records."""
        self.cam = make_camera(camera)
        self.V = int(n_views)
        self.W, self.H = int(camera.width), int(camera.height)
        self.tiles = ((self.W + 15) // 16) * ((self.H + 15) // 16) * self.V
        self.device = torch.device(device)
        self.sched = sched if sched is not None else make_sched()
        self.capacity = int(capacity)
        self.n = -1
        dev = self.device
        VH = self.V * self.H
        self.rgb = torch.empty((3, VH, self.W), dtype=torch.float32, device=dev)
        self.T = torch.empty((VH, self.W), dtype=torch.float32, device=dev)
        self.last = torch.empty((VH, self.W), dtype=torch.int32, device=dev)
        self.pixel_hits = torch.zeros((VH, self.W), dtype=torch.int32, device=dev)
        self.ranges = torch.empty((self.tiles, 2), dtype=torch.int32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.stats = torch.zeros(4, dtype=torch.int64, device=dev)
        self.tile_counts = torch.zeros(self.tiles, dtype=torch.int32, device=dev)
        self.fwd_state = None
        self.plan_ahead = bool(plan_ahead)
        self._plan_pending = False  # a plan built ahead waits for the next forward
        self._pairs_seen = 0  # the last frame's pairs (where its schedule is built)
        self._side = None

    def _ensure(self, n, capacity):
        dev = self.device
        if n != self.n:
            self.splats = torch.empty((max(n, 1), SPLAT_FLOATS), dtype=torch.float32, device=dev)
            self.offsets = torch.empty(n + 1, dtype=torch.int32, device=dev)
            self.grads = torch.empty((max(n, 1), GRAD_FLOATS), dtype=torch.float32, device=dev)
            self.n = n
            self.workspace = None
        if capacity != self.capacity or not hasattr(self, "keys"):
            self.capacity = capacity
            self.keys = torch.empty(max(capacity, 1), dtype=torch.int64, device=dev)
            self.ids = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
            self.sorted_keys = torch.empty(max(capacity, 1), dtype=torch.int64, device=dev)
            self.sorted_ids = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
            self.workspace = None
            self.fwd_state = None
        if self.workspace is None:
            ws = (workspace_size(n, self.W, self.H, self.capacity) if self.V == 1
                  else workspace_size_views(n, self.W, self.H, self.V, self.capacity))
            self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        if self.fwd_state is None:
            fs = (fwd_state_size(self.W, self.H, self.capacity) if self.V == 1
                  else fwd_state_size_views(self.W, self.H, self.V, self.capacity))
            self.fwd_state = torch.empty(fs, dtype=torch.uint8, device=dev)

    def project(self, means, log_scales, quats, opacities, sh, sh_degree):
        """sh as float32, or as bfloat16 (then gs_project_bf16sh reads its bits)."""
        n = int(means.shape[0])
        self._ensure(n, self.capacity)
        call = gs_project_bf16sh if sh.dtype == torch.bfloat16 else gs_project
        call(n, means, log_scales, quats, opacities, sh, sh_degree, self.cam, self.splats)
        return self.splats[:n]

    def enqueue_bin_sort(self, n, want_keys=False, want_emission=False):
        """Enqueue binning and sorting of the current splats (no synchronisation).

        want_emission also writes the id-order (keys, ids) list of gs_bin_tiles;
        want_keys writes the sorted keys."""
        self._ensure(n, self.capacity)
        keys = self.keys if want_emission else None
        ids = self.ids if want_emission else None
        skeys = self.sorted_keys if want_keys else None
        tc = self.tile_counts if self.plan_ahead else None
        if self.V == 1:
            gs_bin_tiles(n, self.splats, self.cam, self.capacity, self.offsets, keys, ids,
                         self.status, self.workspace, tile_counts=tc)
        else:
            gs_bin_tiles_views(n, self.splats, self.cam, self.V, self.capacity, self.offsets,
                               keys, ids, self.status, self.workspace, tile_counts=tc)
        if self.V == 1 and self.plan_ahead and plan_in_sort(self.tiles, self._pairs_seen):
            # the sort builds the schedule in a spare workgroup of its last pass
            gs_sort_keys_plan(n, self.splats, self.offsets, self.capacity, self.cam, skeys,
                              self.sorted_ids, self.ranges, self.sched, self.fwd_state,
                              self.status, self.workspace)
            self._plan_pending = True
            return
        # otherwise the schedule beside the sort, on a second stream
        if self.plan_ahead:
            self._enqueue_plan()
        if self.V == 1:
            gs_sort_keys(n, self.splats, self.offsets, self.capacity, self.cam, skeys,
                         self.sorted_ids, self.ranges, self.status, self.workspace)
        else:
            gs_sort_keys_views(n, self.splats, self.offsets, self.capacity, self.cam, self.V,
                               skeys, self.sorted_ids, self.ranges, self.status, self.workspace)
        if self.plan_ahead:
            torch.cuda.current_stream(self.device).wait_event(self._ev_plan)

    def _enqueue_plan(self):
        """gs_plan_tiles on the side stream, after the binning pass of the current
        stream; the caller makes the current stream wait for self._ev_plan."""
        main = torch.cuda.current_stream(self.device)
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)
            self._ev_bin, self._ev_plan = torch.cuda.Event(), torch.cuda.Event()
        self._ev_bin.record(main)
        self._side.wait_event(self._ev_bin)
        for t in (self.tile_counts, self.fwd_state, self.status):
            t.record_stream(self._side)  # not reused while the side stream may use it
        if self.V == 1:
            gs_plan_tiles(self.tile_counts, self.cam, self.sched, self.fwd_state, self.status,
                          stream=self._side)
        else:
            gs_plan_tiles_views(self.tile_counts, self.cam, self.V, self.sched, self.fwd_state,
                                self.status, stream=self._side)
        self._ev_plan.record(self._side)
        self._plan_pending = True

    def clear_state(self):
        """Zero the forward state (a plan built ahead is dropped with it)."""
        self.fwd_state.zero_()
        self._plan_pending = False

    def _fwd_sched(self):
        """The forward's knobs: with a plan built ahead for this frame, the forward
        checks it inside its own launch (planned)."""
        if not self._plan_pending:
            return self.sched
        self._plan_pending = False
        return planned_sched(self.sched)

    def frame_status(self, n):
        """(device status, pair count I) of the frame, read once (synchronises)."""
        both = torch.cat([self.status, self.offsets[n:n + 1]]).cpu()
        self._pairs_seen = int(both[1])
        return int(both[0]), int(both[1])

    def bin_and_sort(self, n, want_keys=False, want_emission=False):
        """Bin and sort, then read the frame's status once; on a pair overflow grow
        the buffers and run again. Returns I."""
        for _ in range(3):
            self.enqueue_bin_sort(n, want_keys, want_emission)
            st, I = self.frame_status(n)
            if st == GS_OK:
                return I
            if st != GS_ERR_CAPACITY:
                raise GsError(st, "bin_and_sort")
            self._ensure(n, max(I + I // 8, 1024))
        raise GsError(GS_ERR_CAPACITY, "bin_and_sort")

    def render_fwd(self, n, stats=False, background=None, clear_grads=False):
        """Enqueue the forward. stats: also count hits (self.stats, self.pixel_hits,
        both cleared first). background: 3 floats (host), or None for black.
        clear_grads: the forward also clears the gradient rows of the n splats
        (for render_bwd(..., accumulate=True)); one view only."""
        self._ensure(n, self.capacity)
        st = ph = None
        if stats:
            self.stats.zero_()
            self.pixel_hits.zero_()
            st, ph = self.stats, self.pixel_hits
        sched = self._fwd_sched()
        if clear_grads:
            if self.V > 1:
                raise ValueError("clear_grads takes one view")
            gs_render_fwd_zero(n, self.splats, self.sorted_ids, self.ranges, self.cam, sched,
                               self.rgb, self.T, self.last, self.fwd_state, st, ph, self.status,
                               self.grads[:n], background)
            return self.rgb, self.T, self.last
        if self.V > 1:
            gs_render_fwd_views(n, self.splats, self.sorted_ids, self.ranges, self.cam, self.V,
                                sched, self.rgb, self.T, self.last, self.fwd_state, st, ph,
                                self.status, background)
            return self.rgb, self.T, self.last
        args = (n, self.splats, self.sorted_ids, self.ranges, self.cam, sched, self.rgb,
                self.T, self.last, self.fwd_state, st, ph, self.status)
        if background is None:
            gs_render_fwd(*args)
        else:
            gs_render_fwd_bg(*args, background)
        return self.rgb, self.T, self.last

    def render_bwd(self, n, dL_drgb, background=None, dL_dT=None, accumulate=False):
        """Enqueue the backward. background as for render_fwd; dL_dT [H][W] on the
        device, or None. accumulate: add into the gradient rows (cleared by
        render_fwd(..., clear_grads=True) or holding earlier sums)."""
        if accumulate:
            gs_render_bwd_accumulate(n, self.splats, self.sorted_ids, self.ranges, self.cam,
                                     self.V, self.T, self.last, self.fwd_state, dL_drgb,
                                     self.grads, self.status, background, dL_dT)
            return self.grads[:n]
        if self.V > 1:
            gs_render_bwd_views(n, self.splats, self.sorted_ids, self.ranges, self.cam, self.V,
                                self.T, self.last, self.fwd_state, dL_drgb, self.grads,
                                self.status, background, dL_dT)
            return self.grads[:n]
        args = (n, self.splats, self.sorted_ids, self.ranges, self.cam, self.T, self.last,
                self.fwd_state, dL_drgb, self.grads, self.status)
        if background is None and dL_dT is None:
            gs_render_bwd(*args)
        else:
            gs_render_bwd_bg(*args, background, dL_dT)
        return self.grads[:n]

    def check(self, what="frame"):
        """Read the frame's status once and raise GsError unless it is GS_OK."""
        st = int(self.status.cpu()[0])
        if st != GS_OK:
            raise GsError(st, what)

    def run_frame(self, n, dL_drgb=None, stats=False, background=None, dL_dT=None):
        """Bin, sort, forward and (with dL_drgb) backward of the current splats,
        then one read of the frame's status; a pair overflow grows the buffers and
        runs the frame again. Returns I."""
        # one view: the forward clears the gradient rows in its idle end and
        # the backward adds into them (no clearing launch of its own)
        fused = dL_drgb is not None and self.V == 1
        for _ in range(3):
            self.enqueue_bin_sort(n)
            self.render_fwd(n, stats=stats, background=background, clear_grads=fused)
            if dL_drgb is not None:
                self.render_bwd(n, dL_drgb, background=background, dL_dT=dL_dT,
                                accumulate=fused)
            st, I = self.frame_status(n)
            if st == GS_OK:
                return I
            if st != GS_ERR_CAPACITY:
                raise GsError(st, "run_frame")
            self._ensure(n, max(I + I // 8, 1024))
        raise GsError(GS_ERR_CAPACITY, "run_frame")

    def project_bwd(self, means, log_scales, quats, opacities, sh, sh_degree, dL_dsplat=None):
        """Per-Gaussian gradients from the screen-space ones (by default the last
        render_bwd's). Returns a dict of new device tensors."""
        n = int(means.shape[0])
        dsp = self.grads[:n] if dL_dsplat is None else dL_dsplat
        dev = means.device
        K = (int(sh_degree) + 1) ** 2
        out = dict(means=torch.empty((n, 3), dtype=torch.float32, device=dev),
                   log_scales=torch.empty((n, 3), dtype=torch.float32, device=dev),
                   quats=torch.empty((n, 4), dtype=torch.float32, device=dev),
                   opacities=torch.empty(n, dtype=torch.float32, device=dev),
                   sh=torch.empty((n, K, 3), dtype=torch.float32, device=dev))
        call = gs_project_bwd_bf16sh if sh.dtype == torch.bfloat16 else gs_project_bwd
        call(n, means, log_scales, quats, opacities, sh, sh_degree, self.cam, dsp,
             out["means"], out["log_scales"], out["quats"], out["opacities"], out["sh"])
        return out

    def project_views(self, cams, means, log_scales, quats, opacities, sh, sh_degree):
        """Records of every view of the batch (rows [v n, (v + 1) n) for cams[v])."""
        n = int(means.shape[0])
        self._ensure(n * len(cams), self.capacity)
        gs_project_views(n, means, log_scales, quats, opacities, sh, sh_degree, cams, self.splats)
        return self.splats[:n * len(cams)]

    def project_bwd_views(self, cams, means, log_scales, quats, opacities, sh, sh_degree,
                          dL_dsplat=None):
        """Per-Gaussian gradients summed over the views, as a dict of new tensors."""
        n = int(means.shape[0])
        dsp = self.grads[:n * len(cams)] if dL_dsplat is None else dL_dsplat
        dev = means.device
        K = (int(sh_degree) + 1) ** 2
        out = dict(means=torch.empty((n, 3), dtype=torch.float32, device=dev),
                   log_scales=torch.empty((n, 3), dtype=torch.float32, device=dev),
                   quats=torch.empty((n, 4), dtype=torch.float32, device=dev),
                   opacities=torch.empty(n, dtype=torch.float32, device=dev),
                   sh=torch.empty((n, K, 3), dtype=torch.float32, device=dev))
        gs_project_bwd_views(n, means, log_scales, quats, opacities, sh, sh_degree, cams, dsp,
                             out["means"], out["log_scales"], out["quats"], out["opacities"],
                             out["sh"])
        return out
