"""The library's host-side pair grouping (loopvq_tasq_pair_permutation)
against the oracle's, and the argument checks of the two permutation entry
points; no GPU needed."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as ref
import sub_bit_loop_amd as lv
from sub_bit_loop_amd._lib import LoopVQError


def _planted_cov(rng, T_c, D, c, n=2000):
    HD = D // 2
    per = c // 2
    order = rng.permutation(HD)
    k = np.empty((T_c, n, D))
    f = rng.standard_normal((n, HD // per))
    for s in range(T_c):
        if s:
            f = 0.9 * f + np.sqrt(1 - 0.81) * rng.standard_normal(f.shape)
        for gi in range(HD // per):
            for u in order[gi * per:(gi + 1) * per]:
                for ch in (u, u + HD):
                    k[s, :, ch] = rng.uniform(0.5, 2) * f[:, gi] + 0.3 * rng.standard_normal(n)
    y = ref.tasq_scaled_keys(k, rng.lognormal(0, 0.3, D), rng.uniform(0.5, 2, (n, T_c)))
    return ref.stacked_covariance(y)[1]


@pytest.mark.parametrize("T_c,D,c", [(4, 128, 4), (4, 128, 8), (2, 64, 16), (1, 32, 2), (8, 128, 2)])
def test_host_grouping_matches_oracle(T_c, D, c):
    rng = np.random.default_rng(100 + T_c * D + c)
    for cov in (_planted_cov(rng, T_c, D, c),
                ref.stacked_covariance(rng.standard_normal((400, T_c, D)) @ rng.standard_normal((D, D)))[1]):
        want = ref.pair_grouped_permutation(cov, T_c, D, c)
        got = lv.tasq_pair_permutation(torch.from_numpy(np.ascontiguousarray(cov)), T_c, D, c)
        assert got.numpy().astype(np.int64).tolist() == want.tolist()


def test_host_grouping_zero_variance_channels():
    # channels without variance contribute nothing, as in the oracle
    rng = np.random.default_rng(7)
    y = rng.standard_normal((500, 2, 16))
    y[:, :, 3] = 1.5
    y[:, 1, 11] = 0.0
    cov = ref.stacked_covariance(y)[1]
    want = ref.pair_grouped_permutation(cov, 2, 16, 4)
    got = lv.tasq_pair_permutation(torch.from_numpy(cov), 2, 16, 4)
    assert got.numpy().astype(np.int64).tolist() == want.tolist()


def test_permutation_entry_points_reject_bad_arguments():
    L = lv.lib()
    cov = torch.zeros((8, 8), dtype=torch.float64)
    perm = torch.zeros(8, dtype=torch.int16)
    P = ctypes.c_void_p
    assert L.loopvq_tasq_pair_permutation(None, 1, 8, 4, P(perm.data_ptr())) == -1
    assert L.loopvq_tasq_pair_permutation(P(cov.data_ptr()), 1, 8, 3, P(perm.data_ptr())) == -1   # odd c
    assert L.loopvq_tasq_pair_permutation(P(cov.data_ptr()), 1, 8, 6, P(perm.data_ptr())) == -1   # c does not divide D
    assert L.loopvq_tasq_pair_permutation(P(cov.data_ptr()), 0, 8, 4, P(perm.data_ptr())) == -1
    with pytest.raises(LoopVQError):
        lv.tasq_pair_permutation(cov, 1, 7, 2)
    # covariance statistics: validation happens on the host, before any HIP call
    g = lv.geom(128, 4, 4, 16, 256, 1, 1)
    st = (ctypes.c_int64 * 4)(4 * 8 * 128, 4 * 8 * 128, 8 * 128, 128)
    P16 = P(16)
    assert L.loopvq_tasq_covariance(ctypes.byref(g), P16, st, 0, 8, P16, P16, 8, P16, P16, None) == -1
    assert L.loopvq_tasq_covariance(ctypes.byref(g), P16, st, 1, 0, P16, P16, 8, P16, P16, None) == -1
    assert L.loopvq_tasq_covariance(ctypes.byref(g), P16, st, 1, 8, P16, P16, 4, P16, P16, None) == -1  # sig_cap < N
    assert L.loopvq_tasq_covariance(ctypes.byref(g), P16, st, 1, 8, None, P16, 8, P16, P16, None) == -1
    bad = (ctypes.c_int64 * 4)(4 * 8 * 128, 4 * 8 * 128, 8 * 128, 100)
    assert L.loopvq_tasq_covariance(ctypes.byref(g), P16, bad, 1, 8, P16, P16, 8, P16, P16, None) == -1
