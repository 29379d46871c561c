"""Pins of the oracle's covariance-derived, RoPE-pair-grouped channel
permutation (LoopVQ review, section 3.3): a library covariance, a hand-worked
affinity, recovery of planted channel groups, the brute-force best pairing on
tiny inputs, and the structural invariants."""
import numpy as np

import oracle as ref


def _planted(rng, n, T_c, D, c, rho=0.9, noise=0.15):
    """Keys whose RoPE pairs fall into planted groups of c/2 pairs: every
    channel of a group follows the group's own AR(1) factor over the steps.
    Returns k [T_c, n, D] and the planted groups (sets of pair indices)."""
    HD = D // 2
    per = c // 2
    order = rng.permutation(HD)
    groups = [set(order[i:i + per].tolist()) for i in range(0, HD, per)]
    k = np.empty((T_c, n, D))
    f = rng.standard_normal((n, len(groups)))
    load = rng.uniform(0.5, 2.0, size=D) * rng.choice([-1.0, 1.0], size=D)
    for s in range(T_c):
        if s:
            f = rho * f + np.sqrt(1 - rho * rho) * rng.standard_normal(f.shape)
        for gi, g in enumerate(groups):
            for u in g:
                for ch in (u, u + HD):
                    k[s, :, ch] = load[ch] * f[:, gi] + noise * rng.standard_normal(n)
    return k, groups


def _chunks(perm, c):
    return [perm[i:i + c] for i in range(0, len(perm), c)]


def test_stacked_covariance_is_the_library_covariance():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((300, 3, 8)) * rng.uniform(0.1, 3.0, size=8) + 0.7
    mu, cov = ref.stacked_covariance(y)
    Y = y.reshape(300, 24)
    assert np.allclose(mu, Y.mean(axis=0), rtol=0, atol=1e-14)
    assert np.allclose(cov, np.cov(Y, rowvar=False, bias=True), rtol=1e-12, atol=1e-13)


def test_pair_affinity_hand_worked():
    # D = 4: pair 0 = channels {0, 2}, pair 1 = channels {1, 3}; one step.
    corr = np.array([[1.0, 0.5, 0.1, -0.2],
                     [0.5, 1.0, 0.3, 0.0],
                     [0.1, 0.3, 1.0, 0.4],
                     [-0.2, 0.0, 0.4, 1.0]])
    sd = np.array([2.0, 0.5, 1.0, 3.0])
    cov = corr * np.outer(sd, sd)
    A = ref.pair_affinity(cov, 1, 4)
    # |corr(0,1)| + |corr(0,3)| + |corr(2,1)| + |corr(2,3)| = 0.5 + 0.2 + 0.3 + 0.4
    assert np.isclose(A[0, 1], 1.4) and np.isclose(A[1, 0], 1.4)
    assert A[0, 0] == 0 and A[1, 1] == 0


def test_pair_affinity_sums_step_pairs():
    # two steps: the affinity adds the |corr| of every (step, step) combination
    rng = np.random.default_rng(2)
    y = rng.standard_normal((500, 2, 4))
    _, cov = ref.stacked_covariance(y)
    A = ref.pair_affinity(cov, 2, 4)
    corr = np.corrcoef(y.reshape(500, 8), rowvar=False)
    want = sum(abs(corr[s * 4 + a, t * 4 + b]) for s in range(2) for t in range(2) for a in (0, 2) for b in (1, 3))
    assert np.isclose(A[0, 1], want, rtol=1e-12)


def test_planted_groups_are_recovered():
    rng = np.random.default_rng(3)
    for T_c, D, c in [(4, 32, 4), (2, 32, 8), (4, 128, 4), (1, 16, 4)]:
        k, groups = _planted(rng, 3000, T_c, D, c)
        w = rng.lognormal(0.0, 0.3, size=D)
        sig = rng.uniform(0.5, 2.0, size=(3000, T_c))
        y = ref.tasq_scaled_keys(k, w, sig)
        _, cov = ref.stacked_covariance(y)
        perm = ref.pair_grouped_permutation(cov, T_c, D, c)
        got = [set(int(x) for x in ch[0::2]) for ch in _chunks(perm, c)]
        assert sorted(map(sorted, got)) == sorted(map(sorted, groups)), (T_c, D, c)


def test_tiny_inputs_match_the_best_pairing():
    # D = 8: four pairs, c = 4 -> two groups of two pairs; three ways to pair
    # them up.  On planted data the greedy grouping is the best one.
    rng = np.random.default_rng(4)
    for trial in range(5):
        k, _ = _planted(rng, 2000, 2, 8, 4, noise=0.3)
        y = ref.tasq_scaled_keys(k, np.ones(8), np.ones((2000, 2)))
        _, cov = ref.stacked_covariance(y)
        A = ref.pair_affinity(cov, 2, 8)
        best = max(([(0, a), tuple(sorted(set(range(1, 4)) - {a}))] for a in (1, 2, 3)),
                   key=lambda p: A[p[0]] + A[p[1]])
        perm = ref.pair_grouped_permutation(cov, 2, 8, 4)
        got = sorted(tuple(sorted(int(x) for x in ch[0::2])) for ch in _chunks(perm, 4))
        assert got == sorted(best), trial


def test_structure_of_any_permutation():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((800, 4, 128)) @ rng.standard_normal((128, 128)) * 0.1
    _, cov = ref.stacked_covariance(y)
    A = ref.pair_affinity(cov, 4, 128)
    for c in (2, 4, 8, 16):
        perm = ref.pair_grouped_permutation(cov, 4, 128, c)
        assert sorted(perm.tolist()) == list(range(128))
        for ch in _chunks(perm, c):
            # whole RoPE pairs, each written as (u, u + D/2)
            assert all(ch[i + 1] == ch[i] + 64 and ch[i] < 64 for i in range(0, c, 2))
        # the first seed has the largest total affinity
        assert perm[0] == int(np.argmax(A.sum(axis=1)))
        if c == 2:
            # one pair per chunk: pairs in the order of their affinity to the
            # pairs still free when they were picked
            seeds = perm[0::2]
            free = list(range(64))
            for s in seeds:
                tot = A[np.ix_(free, free)].sum(axis=1)
                assert s == free[int(np.argmax(tot))]
                free.remove(s)


def test_identity_scaling_is_invariant():
    # a common positive scale of every key leaves the correlations, and so the
    # permutation, unchanged
    rng = np.random.default_rng(6)
    k, _ = _planted(rng, 1500, 4, 32, 4)
    y1 = ref.tasq_scaled_keys(k, np.ones(32), np.ones((1500, 4)))
    y2 = ref.tasq_scaled_keys(k * 4.0, np.full(32, 0.5), np.full((1500, 4), 2.0))
    p1 = ref.pair_grouped_permutation(ref.stacked_covariance(y1)[1], 4, 32, 4)
    p2 = ref.pair_grouped_permutation(ref.stacked_covariance(y2)[1], 4, 32, 4)
    assert np.array_equal(p1, p2)


def test_scaled_keys_hand_worked():
    # Section 3.3 / eq. (10): weights multiply, the token-step scale divides;
    # sigma differs per token and per step so a swapped or inverted scale fails.
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "tasq_scaled_keys.json")) as f:
        g = json.load(f)
    y = ref.tasq_scaled_keys(np.array(g["k"], float), np.array(g["w"], float),
                             np.array(g["sigma"], float))
    assert np.array_equal(y, np.array(g["y"], float))


def test_scaled_keys_are_the_unpermuted_forward_transform():
    # With the identity permutation the scaled keys are the encode's
    # pre-transformed keys (whose hand-worked case is pinned separately).
    rng = np.random.default_rng(7)
    T_c, n, D = 4, 9, 16
    k = rng.standard_normal((T_c, n, D))
    w = rng.lognormal(0.0, 0.3, size=D)
    sb = rng.uniform(0.25, 4.0, size=(n, T_c))
    y = ref.tasq_scaled_keys(k, w, sb)
    for s in range(T_c):
        z = ref.tasq_forward(k[s], w, np.arange(D), sb[:, s])
        assert np.allclose(y[:, s, :], z, rtol=1e-15, atol=0)
