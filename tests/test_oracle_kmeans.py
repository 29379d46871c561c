"""Pins of the oracle's importance-weighted k-means step (LoopVQ review,
eq. 3): a library weighted Lloyd step, the objective never rising, integer
weights as repeated vectors, invariance to a common weight scale, and the
bf16 rounding against a library conversion."""
import numpy as np
import pytest
import torch

import oracle as ref


def _clustered(rng, n, K, G):
    centres = rng.standard_normal((K, G)) * 4.0
    lab = np.concatenate([np.arange(K), rng.integers(0, K, n - K)])
    z = centres[lab] + 0.3 * rng.standard_normal((n, G))
    init = centres + 0.5 * rng.standard_normal((K, G))
    return z, init


def test_step_is_the_library_weighted_lloyd_step():
    sklearn_cluster = pytest.importorskip("sklearn.cluster")
    rng = np.random.default_rng(11)
    z, init = _clustered(rng, 3000, 12, 16)
    om = rng.lognormal(0.0, 1.0, size=3000)
    a, new = ref.weighted_kmeans_step(z, om, init)
    km = sklearn_cluster.KMeans(n_clusters=12, init=init, n_init=1, max_iter=1, tol=0.0,
                                algorithm="lloyd").fit(z, sample_weight=om)
    assert np.allclose(new, km.cluster_centers_, rtol=1e-10, atol=1e-10)


def test_objective_does_not_rise():
    rng = np.random.default_rng(12)
    z, init = _clustered(rng, 2000, 16, 8)
    om = rng.uniform(0.0, 3.0, size=2000)
    cb = init
    prev = ref.weighted_kmeans_objective(z, om, cb)
    for _ in range(5):
        _, cb = ref.weighted_kmeans_step(z, om, cb)
        cur = ref.weighted_kmeans_objective(z, om, cb)
        assert cur <= prev * (1 + 1e-12)
        prev = cur


def test_integer_weights_are_repeated_vectors():
    rng = np.random.default_rng(13)
    z, init = _clustered(rng, 400, 6, 4)
    om = rng.integers(0, 4, size=400).astype(np.float64)
    _, new_w = ref.weighted_kmeans_step(z, om, init)
    rep = np.repeat(z, om.astype(np.int64), axis=0)
    _, new_r = ref.weighted_kmeans_step(rep, np.ones(len(rep)), init)
    assert np.allclose(new_w, new_r, rtol=1e-13, atol=1e-13)


def test_common_weight_scale_and_empty_codewords():
    rng = np.random.default_rng(14)
    z, init = _clustered(rng, 500, 5, 6)
    init = np.vstack([init, np.full((1, 6), 1e6)])     # a codeword no vector reaches
    om = rng.uniform(0.1, 2.0, size=500)
    a1, n1 = ref.weighted_kmeans_step(z, om, init)
    a2, n2 = ref.weighted_kmeans_step(z, 8.0 * om, init)
    assert np.array_equal(a1, a2) and np.allclose(n1, n2, rtol=1e-14)
    assert np.array_equal(n1[5], init[5])               # zero total weight keeps its value


def test_fisher_weights_sum_all_steps():
    # gradient of one joint vector (G = 4 coordinates over 2 steps): ||g||^2
    g = np.array([[3.0, 0.0, 4.0, 0.0], [1.0, 2.0, 2.0, 4.0]])
    assert np.array_equal(ref.fisher_weights(g), [25.0, 25.0])


def test_bf16_round_is_the_library_conversion():
    rng = np.random.default_rng(15)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, 1.0, -2.5, 1.00390625, 1.01171875, 3.0e38]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ref.bf16_round(x.astype(np.float64)), want)


def test_objective_hand_worked():
    # Eq. 3: each vector's squared distance to its nearest codeword, weighted by
    # its importance.  Two points, one codeword: 2*1^2 + 1*2^2 = 6 (5 unweighted).
    assert ref.weighted_kmeans_objective(np.array([[0.0], [3.0]]), np.array([2.0, 1.0]),
                                         np.array([[1.0]])) == 6.0
    # nearest codeword, not the first: distances 0, 16 (to (3,0)), 49 (to (3,0))
    z = np.array([[0.0, 0.0], [3.0, 4.0], [10.0, 0.0]])
    cb = np.array([[0.0, 0.0], [3.0, 0.0]])
    assert ref.weighted_kmeans_objective(z, np.array([1.0, 2.0, 0.5]), cb) == 56.5
    # zero weight removes a vector's error entirely
    assert ref.weighted_kmeans_objective(z, np.array([0.0, 0.0, 1.0]), cb) == 49.0


def test_objective_integer_weights_are_repeated_vectors():
    rng = np.random.default_rng(16)
    z, init = _clustered(rng, 300, 5, 4)
    om = rng.integers(0, 4, size=300).astype(np.float64)
    rep = np.repeat(z, om.astype(np.int64), axis=0)
    # brute force over the repeated set: min over codewords, summed
    d = ((rep[:, None, :] - init[None, :, :]) ** 2).sum(axis=-1).min(axis=1).sum()
    assert ref.weighted_kmeans_objective(z, om, init) == pytest.approx(d, rel=1e-13)
