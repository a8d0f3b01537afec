"""The give-up path of the bounded device-side waits, forced from the host.

With gs_set_wait_limit(0) every wait that is not satisfied at its first probe
(the sort's look-back over earlier partitions, a chunk's wait for the chunks in
front of it) gives up at once and stores GS_ERR_TIMEOUT: every kernel still
exits normally, the frame's later kernels do nothing (the image keeps what the
caller put there, the gradients are zero), and a frame after the limit is
restored is unaffected. Garden at full size: its 250 depth partitions and 483
tile partitions make look-back waits certain.
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


def test_waits_that_give_up_fail_the_frame_and_nothing_else():
    gsr = _gsr()
    sc = scenegen.make_config(3)
    n = sc.n
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # forced chunks on the heaviest tiles, so the forward has waits as well
    r = gsr.Rasterizer(sc.camera, capacity=1 << 23,
                       sched=gsr.make_sched(chunk_mode=2, force_k=4, force_h=64))
    r.project(up(sc.means), up(sc.log_scales), up(sc.quats), up(sc.opacities), up(sc.sh),
              sc.sh_degree)
    dL = up(sc.dL_drgb)
    r.run_frame(n, dL)
    ref = (r.rgb.cpu().numpy().copy(), r.last.cpu().numpy().copy())
    prev = gsr.gs_set_wait_limit(0)
    try:
        outcomes = []
        for _ in range(3):
            r.status.zero_()
            r.enqueue_bin_sort(n)
            r.rgb.fill_(7.0)
            r.render_fwd(n)
            g = r.render_bwd(n, dL)
            st, _ = r.frame_status(n)
            print("frame with every wait limited to one probe:", gsr.strerror(st), flush=True)
            assert st in (gsr.GS_OK, gsr.GS_ERR_TIMEOUT)
            if st == gsr.GS_ERR_TIMEOUT:
                assert torch.all(g == 0).item()
            outcomes.append(st)
        assert gsr.GS_ERR_TIMEOUT in outcomes
    finally:
        gsr.gs_set_wait_limit(prev)
    r.run_frame(n, dL)
    assert np.array_equal(r.rgb.cpu().numpy(), ref[0])
    assert np.array_equal(r.last.cpu().numpy(), ref[1])
