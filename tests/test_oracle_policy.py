"""Pins of the oracle's per-frame chunking policy: hand-computed cases of the
cost model in "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on
GPUs", section 4.4, Eq. 6 (search k in {2,4,8,16}, chunk only when the
estimate is at least eps = 10% below LPT-only), with exact chunk composition
charged as a second walk of every split tile (avg gains S_h = N_1 + ... + N_h,
the longest unit is 2 N_1 / k). lambda and beta are not printed on the page:
their values stay unpinned; the structure is pinned."""
import numpy as np

import oracle


def test_no_chunking_when_work_dwarfs_the_workers():
    assert oracle.chunk_policy(np.full(1000, 100), workers=10, lambda_=5.0, beta=0.1) == (0, 1)


def test_single_outlier_is_split_sixteen_ways():
    # Ntot = 109990, T0 = max(1099.9, 100000) + 0.1*100000 = 110000.
    # (1,16): l = max(2*100000/16, 10) = 12500, avg = (209990 + 800)/100 = 2107.9
    #   -> 12500 + 1250 = 13750; larger h only ties (same l), smaller k has a larger l.
    counts = np.array([100000] + [10] * 999)
    assert oracle.chunk_policy(counts, workers=100, lambda_=50.0, beta=0.1) == (1, 16)


def test_two_pass_cost_and_ten_percent_threshold():
    # K = 4, lambda = beta = 0. [1000, 800, 790]: Ntot = 2590, T0 = 1000.
    # (1,2): l = 2*1000/2 = 1000 -> no gain; (1,4): l = max(500, 800) = 800,
    # avg = (2590 + 1000)/4 = 897.5 -> 897.5 <= 900; (1,8) only ties -> (1, 4)
    assert oracle.chunk_policy([1000, 800, 790], 4, 0.0, 0.0) == (1, 4)
    # [1000, 820, 800]: avg = (2620 + 1000)/4 = 905 > 900 -> off
    assert oracle.chunk_policy([1000, 820, 800], 4, 0.0, 0.0) == (0, 1)


def test_chunk_overhead_term_picks_k():
    # two outliers of 8000 among 200 tiles of 100: Ntot = 36000, K = 8, beta = 0.5,
    # T0 = 8000 + 4000 = 12000 (threshold 10800). h = 1 keeps l = N_2 = 8000.
    counts = np.array([8000, 8000] + [100] * 200)
    # lambda = 0: (2,16): l = max(1000, 100), avg = (36000 + 16000)/8 = 6500 -> 7000;
    #   (2,8) -> 6500 + 1000, (2,4) -> 6500 + 2000
    assert oracle.chunk_policy(counts, workers=8, lambda_=0.0, beta=0.5) == (2, 16)
    # lambda = 400: (2,4): (52000 + 3200)/8 + 2000 = 8900; (2,8): (52000 + 6400)/8 + 1000
    #   = 8300; (2,16): (52000 + 12800)/8 + 500 = 8600 -> (2, 8)
    assert oracle.chunk_policy(counts, workers=8, lambda_=400.0, beta=0.5) == (2, 8)
    # lambda = 1000, beta = 0: T0 = 8000; (2,4): (52000 + 8000)/8 = 7500 > 7200 -> off
    assert oracle.chunk_policy(counts, workers=8, lambda_=1000.0, beta=0.0) == (0, 1)


def test_empty_and_zero_frames():
    assert oracle.chunk_policy(np.zeros(0, np.int32), 10, 1.0, 0.1) == (0, 1)
    assert oracle.chunk_policy(np.zeros(16, np.int32), 10, 1.0, 0.1) == (0, 1)
