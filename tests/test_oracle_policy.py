"""Pins of the oracle's per-frame chunking policy: hand-computed cases of the
cost model in "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on
GPUs", section 4.4, Eq. 6 (search k in {2,4,8,16}, chunk only when the
estimate is at least eps = 10% below LPT-only). lambda and beta are not
printed on the page: their values stay unpinned; the structure is pinned."""
import numpy as np

import oracle


def test_no_chunking_when_work_dwarfs_the_workers():
    assert oracle.chunk_policy(np.full(1000, 100), workers=10, lambda_=5.0, beta=0.1) == (0, 1)


def test_single_outlier_is_split_sixteen_ways():
    # T0 = max(109990/100, 100000) + 0.1*100000 = 110000; (1,16): l = 6250 -> 6875
    counts = np.array([100000] + [10] * 999)
    assert oracle.chunk_policy(counts, workers=100, lambda_=50.0, beta=0.1) == (1, 16)


def test_ten_percent_threshold_and_first_minimum():
    # K=4, lambda=beta=0: T0 = 1000; best (h=2,k=2) = max(3610/4, 900) = 902.5 > 900 -> off
    assert oracle.chunk_policy([1000, 910, 900, 800], 4, 0.0, 0.0) == (0, 1)
    # T0 = 1010; best = max(3620/4, 900) = 905 <= 909 -> (2, 2); h=3 ties and loses
    assert oracle.chunk_policy([1010, 910, 900, 800], 4, 0.0, 0.0) == (2, 2)


def test_chunk_overhead_term_limits_h():
    # a large lambda makes every extra chunk expensive. Ntot = 29000, K = 8, T0 = 5000;
    # (1,2): max((29000+4000)/8, max(2500, 4000)) = 4125; (2,2) and (1,4): 4625
    counts = np.array([5000, 4000] + [100] * 200)
    assert oracle.chunk_policy(counts, workers=8, lambda_=2000.0, beta=0.0) == (1, 2)
    # with free chunks the second outlier is split too: (2,2) -> max(29000/8, 2500) = 3625;
    # (2,4) only ties it, and the first strict minimum is kept
    assert oracle.chunk_policy(counts, workers=8, lambda_=0.0, beta=0.0) == (2, 2)


def test_empty_and_zero_frames():
    assert oracle.chunk_policy(np.zeros(0, np.int32), 10, 1.0, 0.1) == (0, 1)
    assert oracle.chunk_policy(np.zeros(16, np.int32), 10, 1.0, 0.1) == (0, 1)
