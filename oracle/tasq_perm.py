"""Plain fp64 definition of the pre-transform's channel permutation derived
from the stacked-step covariance, keeping RoPE pairs together.

TEST INFRASTRUCTURE: imported only by tests, smoke() and the benchmark's
CPU-baseline leg.

Source: the LoopVQ review page (jaehun.me, "paper-2611-05304v1"), section 3.3:
the permutation P is taken from the covariance of the T_c step keys of a
block stacked into one T_c*D vector, and each step's RoPE pair {i, i + D/2}
is kept inside one group, so that a group holds c channels (c/2 pairs) per
step and G = c*T_c coordinates; the aim of the transform is that channels
sharing a code are strongly correlated.

Readings taken where the page is silent (listed with their reasons in the
design notes of the repository):
  * the covariance is of the scaled keys y = w * k / sigma_bar (the transform
    before its permutation), centred, normalised by the token count n;
  * pairs are grouped by the magnitude of their correlation: the affinity of
    pairs u and v is the sum of |corr| over both channels of each pair and
    every (step, step) combination of the block, evaluated for u < v and used
    for both orders;
  * groups are formed greedily, one at a time: the seed is the free pair with
    the largest affinity to all other free pairs, then the free pair with the
    largest summed affinity to the group's members joins, until the group has
    c/2 pairs; ties go to the lowest pair index;
  * chunk q is the q-th group formed; inside it the pairs keep the order in
    which they joined, each written as (u, u + D/2).
"""
import numpy as np


def tasq_scaled_keys(k_blk: np.ndarray, w: np.ndarray, sigma_bar: np.ndarray) -> np.ndarray:
    """k_blk [T_c, n, D] raw keys of one (kv-head, block) over n tokens,
    w [D], sigma_bar [n, T_c] -> y [n, T_c, D] = w * k / sigma_bar."""
    k = np.asarray(k_blk, dtype=np.float64)
    y = np.asarray(w, dtype=np.float64)[None, None, :] * k / np.asarray(sigma_bar, dtype=np.float64).T[:, :, None]
    return np.transpose(y, (1, 0, 2))


def stacked_covariance(y: np.ndarray):
    """y [n, T_c, D] -> (mean [T_c*D], covariance [T_c*D, T_c*D]) with the
    step-major feature index s*D + d, centred, divided by n."""
    n = y.shape[0]
    Y = np.asarray(y, dtype=np.float64).reshape(n, -1)
    mu = Y.mean(axis=0)
    Yc = Y - mu
    return mu, (Yc.T @ Yc) / n


def pair_affinity(cov: np.ndarray, T_c: int, D: int) -> np.ndarray:
    """Affinity of RoPE pairs u, v < D/2: sum of |corr| between the channels
    {u, u + D/2} and {v, v + D/2} over all (step, step) pairs; zero diagonal."""
    cov = np.asarray(cov, dtype=np.float64)
    sd = np.sqrt(np.maximum(np.diag(cov), 0.0))
    with np.errstate(divide="ignore", invalid="ignore"):
        corr = cov / np.outer(sd, sd)
    corr[~np.isfinite(corr)] = 0.0
    HD = D // 2
    a = np.abs(corr).reshape(T_c, D, T_c, D)
    # fold the steps and the two channels of each pair
    a = a.sum(axis=(0, 2))                                  # [D, D]
    A = a[:HD, :HD] + a[:HD, HD:] + a[HD:, :HD] + a[HD:, HD:]
    # defined once per unordered pair (from u < v), so that ties which are
    # exact in real arithmetic stay exact
    iu = np.triu_indices(HD, 1)
    A[(iu[1], iu[0])] = A[iu]
    np.fill_diagonal(A, 0.0)
    return A


def pair_grouped_permutation(cov: np.ndarray, T_c: int, D: int, c: int) -> np.ndarray:
    """Permutation p [D] (transformed channel d' holds raw channel p[d'])
    whose chunks of c channels each hold c/2 whole RoPE pairs."""
    assert c % 2 == 0 and D % c == 0
    A = pair_affinity(cov, T_c, D)
    HD = D // 2
    per = c // 2
    free = list(range(HD))
    perm = []
    while free:
        fa = np.array(free)
        tot = A[np.ix_(fa, fa)].sum(axis=1)
        seed = free[int(np.argmax(tot))]                    # argmax: first maximum = lowest index
        group = [seed]
        free.remove(seed)
        while len(group) < per:
            fa = np.array(free)
            gain = A[np.ix_(fa, np.array(group))].sum(axis=1)
            nxt = free[int(np.argmax(gain))]
            group.append(nxt)
            free.remove(nxt)
        for u in group:
            perm += [u, u + HD]
    return np.asarray(perm, dtype=np.int64)
