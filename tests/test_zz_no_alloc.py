"""The allocation-free sort (gs_sort_keys_noalloc) against the sort with a
caller's workspace (gs_bin_tiles + gs_sort_keys), through the C ABI.

Both run the same kernels; the allocation-free call keeps their workspace in
the library's static per-GPU array instead. Pair offsets, the device status,
sorted ids, sorted keys and tile ranges must agree bit for bit, on two calls in
a row (the second with a smaller frame, so the array holds the first call's
state when it starts), and a frame too large for the array must be refused
before any work is enqueued.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import scenegen

pytestmark = pytest.mark.gpu


def _gsr():
    import gaussian_splatting_differentiable_amd as gsr
    gsr.lib()
    return gsr


def _splats(gsr, sc):
    r = gsr.Rasterizer(sc.camera, capacity=16)
    d = [torch.from_numpy(np.ascontiguousarray(a)).cuda()
         for a in (sc.means, sc.log_scales, sc.quats, sc.opacities, sc.sh)]
    return r.project(*d, sc.sh_degree).clone()


def _with_workspace(gsr, sc, splats, cap):
    """gs_bin_tiles + gs_sort_keys with a workspace the caller allocates."""
    cam = gsr.make_camera(sc.camera)
    n = sc.n
    dev = splats.device
    out = dict(offsets=torch.empty(n + 1, dtype=torch.int32, device=dev),
               status=torch.empty(1, dtype=torch.int32, device=dev),
               sorted_ids=torch.empty(cap, dtype=torch.int32, device=dev),
               sorted_keys=torch.empty(cap, dtype=torch.int64, device=dev),
               ranges=torch.empty((sc.camera.num_tiles, 2), dtype=torch.int32, device=dev))
    ws = torch.empty(gsr.workspace_size(n, sc.camera.width, sc.camera.height, cap),
                     dtype=torch.uint8, device=dev)
    gsr.gs_bin_tiles(n, splats, cam, cap, out["offsets"], None, None, out["status"], ws)
    gsr.gs_sort_keys(n, splats, out["offsets"], cap, cam, out["sorted_keys"], out["sorted_ids"],
                     out["ranges"], out["status"], ws)
    return out


def _noalloc(gsr, sc, splats, cap):
    cam = gsr.make_camera(sc.camera)
    n = sc.n
    dev = splats.device
    out = dict(offsets=torch.full((n + 1,), -9, dtype=torch.int32, device=dev),
               status=torch.full((1,), -9, dtype=torch.int32, device=dev),
               sorted_ids=torch.full((cap,), -9, dtype=torch.int32, device=dev),
               sorted_keys=torch.full((cap,), -9, dtype=torch.int64, device=dev),
               ranges=torch.full((sc.camera.num_tiles, 2), -9, dtype=torch.int32, device=dev))
    gsr.gs_sort_keys_noalloc(n, splats, cam, cap, out["offsets"], out["sorted_keys"],
                             out["sorted_ids"], out["ranges"], out["status"])
    return out


def _same(a, b):
    torch.cuda.synchronize()
    st = int(a["status"].cpu()[0])
    assert st == int(b["status"].cpu()[0]) == 0
    I = int(a["offsets"][-1].cpu())
    assert I == int(b["offsets"][-1].cpu()) and I > 0
    assert torch.equal(a["offsets"], b["offsets"])
    assert torch.equal(a["ranges"], b["ranges"])
    assert torch.equal(a["sorted_ids"][:I], b["sorted_ids"][:I])
    assert torch.equal(a["sorted_keys"][:I], b["sorted_keys"][:I])
    return I


def test_noalloc_sort_equals_workspace_sort_twice_second_smaller():
    gsr = _gsr()
    big = scenegen.make_config(2)                                    # 100k Gaussians, 256x256
    small = scenegen.random_scene(501, 3000, 83, 45, 75.0, degree=1, log_scale=(-2.0, 0.6),
                                  opacity=(1.0, 2.0))
    for sc, cap in ((big, 300_000), (small, 40_000)):
        assert gsr.workspace_size(sc.n, sc.camera.width, sc.camera.height, cap) <= \
            gsr.NOALLOC_SCRATCH_BYTES
        sp = _splats(gsr, sc)
        ref = _with_workspace(gsr, sc, sp, cap)
        got = _noalloc(gsr, sc, sp, cap)
        I = _same(got, ref)
        print(f"{sc.name}: {I} pairs equal", flush=True)


def test_noalloc_sort_reports_overflow_like_the_workspace_sort():
    gsr = _gsr()
    sc = scenegen.make_config(1)
    sp = _splats(gsr, sc)
    got = _noalloc(gsr, sc, sp, 64)                                  # far too few pairs
    torch.cuda.synchronize()
    assert int(got["status"].cpu()[0]) == gsr.GS_ERR_CAPACITY
    assert torch.all(got["ranges"] == 0)
    ref = _with_workspace(gsr, sc, sp, 4096)
    got = _noalloc(gsr, sc, sp, 4096)                                # and the next call recovers
    _same(got, ref)


def test_noalloc_sort_refuses_frames_beyond_its_array():
    gsr = _gsr()
    sc = scenegen.make_config(1)
    cam = gsr.make_camera(sc.camera)
    dev = torch.device("cuda")
    n, cap = 3_000_000, 8_000_000
    assert gsr.workspace_size(n, sc.camera.width, sc.camera.height, cap) > gsr.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.int32, device=dev)
    with pytest.raises(gsr.GsError) as e:
        gsr.gs_sort_keys_noalloc(n, torch.zeros((1, 12), device=dev), cam, cap, x, None, x, x, x)
    assert e.value.status == gsr.GS_ERR_WORKSPACE
