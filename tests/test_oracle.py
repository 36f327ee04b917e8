"""The CPU oracle against facts fixed by the pages and by mathematics."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("threads", [1, 2, 3, 8, 64])
def test_threaded_oracle_equals_plain(threads):
    # the all-cores CPU baseline runs the oracle with its rows split over
    # threads; every split must give the plain oracle's result
    import numpy as np
    import oracle
    import workloads
    for (M, K, N) in [(37, 300, 5), (1, 64, 1), (100, 1000, 3), (0, 5, 2), (7, 0, 2), (130, 65, 32)]:
        p = workloads.random_int4_problem(M + K, M, K, N)
        s = oracle.encode(p.W)
        Xp = pins._pack_x_for_test(p.X)
        assert np.array_equal(oracle.spmm_w4a4(s, Xp, N), oracle.spmm_w4a4(s, Xp, N, threads=threads))
        q = workloads.random_fp16_problem(M + K, M, K, N)
        s = oracle.encode(q.W)
        assert np.array_equal(oracle.spmm_f16(s, q.X), oracle.spmm_f16(s, q.X, threads=threads))
