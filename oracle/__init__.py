"""CPU oracle for the differentiable Gaussian-splatting rasterizer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark are the only callers. The product path (the HIP library and
its binding) never imports this package, and this package imports nothing from
the product path; the two share only the seeded input generator ``scenegen``.

The C sources next to this file are the oracle proper (plain, slow, fp64 where
values matter, canonical fp32 where decisions must match bit for bit). This
module compiles them with gcc and exposes numpy-friendly wrappers.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SOURCES = ["project.c", "bin.c", "sort.c", "render.c", "sched.c"]
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp32 mirror needs -ffp-contract=off)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    srcs = [os.path.join(_HERE, s) for s in _SOURCES]
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
           "-Wall", "-Wno-unknown-pragmas", "-o", tmp] + srcs + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Camera(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32),
                ("fx", C.c_double), ("fy", C.c_double), ("cx", C.c_double), ("cy", C.c_double),
                ("w2c", C.c_double * 12), ("znear", C.c_double), ("lowpass", C.c_double)]


def _camera(cam) -> Camera:
    c = Camera()
    c.width, c.height = int(cam.width), int(cam.height)
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    for i, v in enumerate(np.asarray(cam.world_to_cam, np.float64).reshape(12)):
        c.w2c[i] = float(v)
    c.znear, c.lowpass = float(cam.znear), float(cam.lowpass)
    return c


def _load():
    global _lib
    if _lib is not None:
        return _lib
    newest_src = max(os.path.getmtime(os.path.join(_HERE, s)) for s in _SOURCES + ["oracle.h"])
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest_src:
        build()
    lib = C.CDLL(_LIB_PATH)
    P = C.c_void_p
    i32, i64, dbl = C.c_int32, C.c_int64, C.c_double
    sig = {
        "or_sh_basis": [i32, P, P],
        "or_project": [i32, P, P, P, P, P, i32, C.POINTER(Camera), P, P],
        "or_project64": [i32, P, P, P, P, P, i32, C.POINTER(Camera), P],
        "or_sh_cart": [i32, P, P, P],
        "or_project_bwd": [i32, P, P, P, P, P, i32, C.POINTER(Camera), P, P, P, P, P, P],
        "or_bin_count": [i32, P, i32, i32, P],
        "or_bin_emit": [i32, P, i32, i32, P, P, P],
        "or_sort_pairs": [i64, P, P, P, P],
        "or_tile_ranges": [i64, P, i32, P],
        "or_render_fwd": [P, P, P, i32, i32, P, P, P, P, P, P, P, P, P],
        "or_render_fwd_untiled": [i32, P, i32, i32, P, P, P],
        "or_render_fwd_values": [P, P, P, P, i32, i32, P, P, P, P],
        "or_render_bwd": [P, P, P, i32, i32, P, P, P, P, i32, P],
        "or_chunk_policy": [i32, P, dbl, dbl, dbl, dbl, i32, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.or_num_threads.argtypes, lib.or_num_threads.restype = [], C.c_int
    lib.or_set_num_threads.argtypes, lib.or_set_num_threads.restype = [C.c_int], None
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().or_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's later parallel loops."""
    _load().or_set_num_threads(int(n))


def sh_basis(degree: int, d) -> np.ndarray:
    d = _c(d, np.float64)
    out = np.zeros(16, np.float64)
    _load().or_sh_basis(degree, _p(d), _p(out))
    return out[: (degree + 1) ** 2]


def project(means, log_scales, quats, opacities, sh, sh_degree, camera, want_f64=False):
    lib = _load()
    means, log_scales, quats = _c(means, np.float32), _c(log_scales, np.float32), _c(quats, np.float32)
    opacities, sh = _c(opacities, np.float32), _c(sh, np.float32)
    n = means.shape[0]
    out = np.zeros((n, 12), np.float32)
    out64 = np.zeros((n, 12), np.float64) if want_f64 else None
    cam = _camera(camera)
    lib.or_project(n, _p(means), _p(log_scales), _p(quats), _p(opacities), _p(sh),
                   int(sh_degree), C.byref(cam), _p(out), _p(out64))
    return (out, out64) if want_f64 else out


def project64(means, log_scales, quats, opacities, sh, sh_degree, camera):
    """The projection on fp64 inputs; fp64 records (for finite differences)."""
    args = [_c(a, np.float64) for a in (means, log_scales, quats, opacities, sh)]
    n = args[0].shape[0]
    out = np.zeros((n, 12), np.float64)
    cam = _camera(camera)
    _load().or_project64(n, *[_p(a) for a in args], int(sh_degree), C.byref(cam), _p(out))
    return out


def sh_cart(degree: int, d):
    """The SH basis as polynomials of the direction and their gradients."""
    d = _c(d, np.float64)
    Y = np.zeros(16, np.float64)
    dY = np.zeros((16, 3), np.float64)
    _load().or_sh_cart(degree, _p(d), _p(Y), _p(dY))
    K = (degree + 1) ** 2
    return Y[:K], dY[:K]


def project_bwd(means, log_scales, quats, opacities, sh, sh_degree, camera, dsplat):
    """Backward of the projection in fp64: dL/d(means, log_scales, quats,
    opacities, sh) from dL/d of the records' first nine entries."""
    lib = _load()
    means, log_scales, quats = _c(means, np.float32), _c(log_scales, np.float32), _c(quats, np.float32)
    opacities, sh = _c(opacities, np.float32), _c(sh, np.float32)
    n = means.shape[0]
    K = (sh_degree + 1) ** 2
    dsplat = _c(np.asarray(dsplat)[:, :9], np.float64)
    out = dict(means=np.zeros((n, 3)), log_scales=np.zeros((n, 3)), quats=np.zeros((n, 4)),
               opacities=np.zeros(n), sh=np.zeros((n, K, 3)))
    cam = _camera(camera)
    lib.or_project_bwd(n, _p(means), _p(log_scales), _p(quats), _p(opacities), _p(sh),
                       int(sh_degree), C.byref(cam), _p(dsplat), _p(out["means"]),
                       _p(out["log_scales"]), _p(out["quats"]), _p(out["opacities"]), _p(out["sh"]))
    return out


def project_scene(scene, want_f64=False):
    return project(scene.means, scene.log_scales, scene.quats, scene.opacities, scene.sh,
                   scene.sh_degree, scene.camera, want_f64)


def bin_counts(splats, width, height) -> np.ndarray:
    splats = _c(splats, np.float32)
    counts = np.zeros(splats.shape[0], np.int32)
    _load().or_bin_count(splats.shape[0], _p(splats), int(width), int(height), _p(counts))
    return counts


def bin_tiles(splats, width, height):
    """Returns (offsets int64[n+1], keys uint64[I], ids int32[I]) in emission order."""
    splats = _c(splats, np.float32)
    n = splats.shape[0]
    counts = bin_counts(splats, width, height)
    offsets = np.zeros(n + 1, np.int64)
    np.cumsum(counts, out=offsets[1:])
    npairs = int(offsets[-1])
    keys = np.zeros(max(npairs, 1), np.uint64)
    ids = np.zeros(max(npairs, 1), np.int32)
    _load().or_bin_emit(n, _p(splats), int(width), int(height), _p(offsets), _p(keys), _p(ids))
    return offsets, keys[:npairs], ids[:npairs]


def sort_pairs(keys, ids):
    keys, ids = _c(keys, np.uint64), _c(ids, np.int32)
    npairs = keys.shape[0]
    sk = np.zeros(max(npairs, 1), np.uint64)
    si = np.zeros(max(npairs, 1), np.int32)
    _load().or_sort_pairs(npairs, _p(keys), _p(ids), _p(sk), _p(si))
    return sk[:npairs], si[:npairs]


def tile_ranges(sorted_keys, ntiles) -> np.ndarray:
    sorted_keys = _c(sorted_keys, np.uint64)
    ranges = np.zeros((ntiles, 2), np.int32)
    _load().or_tile_ranges(sorted_keys.shape[0], _p(sorted_keys), int(ntiles), _p(ranges))
    return ranges


def _bg(bg, dtype):
    return None if bg is None else np.ascontiguousarray(np.asarray(bg, dtype).reshape(3))


def render_fwd(splats, sorted_ids, ranges, width, height, tile_mask=None, bg=None):
    """Mirror forward (bg: background colour, black when None).
    Returns dict(rgb[3,H,W], T[H,W], last[H,W], knife[H,W], hits, evals,
    pixel_hits[H,W] (splats blended per pixel), pair_quarters[I] (bit q: some
    pixel of quarter q of the pair's tile blended it))."""
    splats, sorted_ids = _c(splats, np.float32), _c(sorted_ids, np.int32)
    ranges = _c(ranges, np.int32)
    rgb = np.zeros((3, height, width), np.float32)
    T = np.zeros((height, width), np.float32)
    last = np.zeros((height, width), np.int32)
    knife = np.zeros((height, width), np.uint8)
    pixel_hits = np.zeros((height, width), np.int32)
    npairs = int(ranges[-1, 1]) if len(ranges) else 0
    pq = np.zeros(max(npairs, 1), np.uint8)
    stats = np.zeros(2, np.int64)
    mask = _c(tile_mask, np.uint8) if tile_mask is not None else None
    bg = _bg(bg, np.float32)
    _load().or_render_fwd(_p(splats), _p(sorted_ids), _p(ranges), int(width), int(height),
                          _p(mask), _p(bg), _p(rgb), _p(T), _p(last), _p(knife), _p(stats),
                          _p(pixel_hits), _p(pq))
    return dict(rgb=rgb, T=T, last=last, knife=knife.astype(bool), hits=int(stats[0]),
                evals=int(stats[1]), pixel_hits=pixel_hits, pair_quarters=pq[:npairs])


def render_fwd_untiled(splats, width, height, want_hits=False):
    """Every pixel over every visible splat in (depth, id) order: (rgb, T), plus
    the per-pixel hit counts when want_hits."""
    splats = _c(splats, np.float32)
    rgb = np.zeros((3, height, width), np.float32)
    T = np.zeros((height, width), np.float32)
    hits = np.zeros((height, width), np.int32)
    _load().or_render_fwd_untiled(splats.shape[0], _p(splats), int(width), int(height),
                                  _p(rgb), _p(T), _p(hits))
    return (rgb, T, hits) if want_hits else (rgb, T)


def render_fwd_values(splats_dec, splats_val, sorted_ids, ranges, width, height, last, bg=None):
    splats_dec, splats_val = _c(splats_dec, np.float32), _c(splats_val, np.float64)
    sorted_ids, ranges, last = _c(sorted_ids, np.int32), _c(ranges, np.int32), _c(last, np.int32)
    rgb = np.zeros((3, height, width), np.float64)
    T = np.zeros((height, width), np.float64)
    bg = _bg(bg, np.float64)
    _load().or_render_fwd_values(_p(splats_dec), _p(splats_val), _p(sorted_ids), _p(ranges),
                                 int(width), int(height), _p(last), _p(bg), _p(rgb), _p(T))
    return rgb, T


def render_bwd(splats, sorted_ids, ranges, width, height, last, dL_drgb, bg=None,
               dL_dT=None) -> np.ndarray:
    """grads[n][9] of sum(dL_drgb * rgb) + sum(dL_dT * T) (bg: background colour)."""
    splats, sorted_ids = _c(splats, np.float32), _c(sorted_ids, np.int32)
    ranges, last, dL = _c(ranges, np.int32), _c(last, np.int32), _c(dL_drgb, np.float32)
    bg = _bg(bg, np.float32)
    dT = None if dL_dT is None else _c(dL_dT, np.float32)
    n = splats.shape[0]
    grads = np.zeros((n, 9), np.float64)
    _load().or_render_bwd(_p(splats), _p(sorted_ids), _p(ranges), int(width), int(height),
                          _p(last), _p(dL), _p(bg), _p(dT), n, _p(grads))
    return grads


def chunk_policy(counts_desc, workers, lambda_, beta, eps=0.10, max_items=1 << 30):
    counts_desc = _c(counts_desc, np.int32)
    h = np.zeros(1, np.int32)
    k = np.zeros(1, np.int32)
    _load().or_chunk_policy(counts_desc.shape[0], _p(counts_desc), float(workers),
                            float(lambda_), float(beta), float(eps), int(max_items), _p(h), _p(k))
    return int(h[0]), int(k[0])


def frame(scene, fwd=True, bwd=True, bg=None, dL_dT=None):
    """Whole oracle chain on a scene: project, bin, sort, ranges, forward, backward
    (bg: background colour; dL_dT: gradient of the final transmittance)."""
    cam = scene.camera
    W, H = cam.width, cam.height
    splats = project_scene(scene)
    offsets, keys, ids = bin_tiles(splats, W, H)
    skeys, sids = sort_pairs(keys, ids)
    ranges = tile_ranges(skeys, cam.num_tiles)
    out = dict(splats=splats, offsets=offsets, keys=keys, ids=ids, sorted_keys=skeys,
               sorted_ids=sids, ranges=ranges)
    if fwd:
        out["fwd"] = render_fwd(splats, sids, ranges, W, H, bg=bg)
    if fwd and bwd:
        out["grads"] = render_bwd(splats, sids, ranges, W, H, out["fwd"]["last"], scene.dL_drgb,
                                  bg=bg, dL_dT=dL_dT)
    return out


def frame_views(scene, cams, dL_drgbs, bg=None, dL_dTs=None):
    """A batch of views as the batch calls lay it out, built from one oracle frame
    per view: view v's records are rows [v n, (v + 1) n) with v in their pad word,
    its tiles follow the tiles of the views before it, its pixels their rows.
    dL_drgbs[v] [3][H][W] and dL_dTs[v] [H][W] (or None) are view v's gradients."""
    import dataclasses
    n = scene.n
    per = []
    for v, cam in enumerate(cams):
        sc = dataclasses.replace(scene, camera=cam, dL_drgb=dL_drgbs[v])
        per.append(frame(sc, bg=bg, dL_dT=None if dL_dTs is None else dL_dTs[v]))
    T1 = cams[0].num_tiles
    splats, offs, keys, ids, skeys, sids, ranges = [], [], [], [], [], [], []
    base = 0
    for v, f in enumerate(per):
        s = f["splats"].copy()
        s[:, 11] = np.array([v], np.int32).view(np.float32)[0]
        splats.append(s)
        offs.append(f["offsets"][:-1] + base)
        shift = np.uint64(v * T1) << np.uint64(32)
        keys.append(f["keys"] + shift)
        ids.append(f["ids"] + v * n)
        skeys.append(f["sorted_keys"] + shift)
        sids.append(f["sorted_ids"] + v * n)
        ranges.append(f["ranges"] + base)
        base += len(f["ids"])
    out = dict(splats=np.concatenate(splats), offsets=np.concatenate(offs + [np.array([base])]),
               keys=np.concatenate(keys), ids=np.concatenate(ids).astype(np.int32),
               sorted_keys=np.concatenate(skeys), sorted_ids=np.concatenate(sids).astype(np.int32),
               ranges=np.concatenate(ranges).astype(np.int32))
    if "fwd" in per[0]:
        fw = [f["fwd"] for f in per]
        out["fwd"] = dict(rgb=np.concatenate([f["rgb"] for f in fw], axis=1),
                          T=np.concatenate([f["T"] for f in fw]),
                          last=np.concatenate([f["last"] for f in fw]),
                          knife=np.concatenate([f["knife"] for f in fw]),
                          pixel_hits=np.concatenate([f["pixel_hits"] for f in fw]),
                          pair_quarters=np.concatenate([f["pair_quarters"] for f in fw]),
                          hits=sum(f["hits"] for f in fw), evals=sum(f["evals"] for f in fw))
    if "grads" in per[0]:
        out["grads"] = np.concatenate([f["grads"] for f in per])
    return out
