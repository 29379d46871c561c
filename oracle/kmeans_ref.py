"""Plain fp64 definition of one step of the importance-weighted (Fisher)
k-means that produces the codebooks.

TEST INFRASTRUCTURE: imported only by tests, smoke() and the benchmark's
CPU-baseline leg.

Source: the LoopVQ review page (jaehun.me, "paper-2611-05304v1"):
  * "codebook and calibration" (eq. 3): the codebook is built offline by
    k-means in which each joint vector n is weighted by its importance
    omega_n = ||dL/dz_n||^2, the squared gradient norm of the next-token loss
    (the diagonal of the empirical Fisher information);
  * section 3.1: for a loop-axis joint vector the weight sums the squared
    gradients of all T_c steps the vector covers.

Readings taken where the page is silent (listed with their reasons in the
design notes of the repository):
  * one step is the usual Lloyd step of a weighted k-means: assign every joint
    vector to its nearest codeword (the same exact argmin as the encode, the
    weights do not enter it), then move each codeword to the weighted mean
    sum_n omega_n z_n / sum_n omega_n of its vectors;
  * a codeword with zero total weight keeps its value;
  * the codebook is stored as bf16, rounded to nearest even.
"""
import numpy as np

from .loopvq_ref import nearest_codeword


def fisher_weights(grad_joint: np.ndarray) -> np.ndarray:
    """grad_joint [..., G]: gradient of the loss w.r.t. each joint vector (its
    G coordinates cover the T_c steps) -> omega [...] = ||grad||^2."""
    g = np.asarray(grad_joint, dtype=np.float64)
    return (g * g).sum(axis=-1)


def weighted_kmeans_sums(z: np.ndarray, omega: np.ndarray, cb: np.ndarray, assign=None):
    """z [n, G], omega [n] >= 0, cb [K, G] -> (assignment [n],
    sums [K, G] = sum of omega z per codeword, wsum [K] = sum of omega).
    `assign`, when given, replaces the argmin (to compare an update made
    from the same assignment)."""
    z = np.asarray(z, dtype=np.float64)
    om = np.asarray(omega, dtype=np.float64)
    a = nearest_codeword(z, cb)[0] if assign is None else np.asarray(assign, dtype=np.int64)
    K, G = np.asarray(cb).shape
    sums = np.zeros((K, G))
    wsum = np.zeros(K)
    np.add.at(sums, a, om[:, None] * z)
    np.add.at(wsum, a, om)
    return a, sums, wsum


def weighted_kmeans_step(z: np.ndarray, omega: np.ndarray, cb: np.ndarray):
    """One weighted Lloyd step.  Returns (assignment, new codebook fp64 [K, G])."""
    cb = np.asarray(cb, dtype=np.float64)
    a, sums, wsum = weighted_kmeans_sums(z, omega, cb)
    new = cb.copy()
    nz = wsum > 0
    new[nz] = sums[nz] / wsum[nz, None]
    return a, new


def weighted_kmeans_objective(z: np.ndarray, omega: np.ndarray, cb: np.ndarray) -> float:
    """sum_n omega_n min_r ||z_n - e_r||^2."""
    z = np.asarray(z, dtype=np.float64)
    cb = np.asarray(cb, dtype=np.float64)
    a, _ = nearest_codeword(z, cb)
    d = z - cb[a]
    return float((np.asarray(omega, dtype=np.float64) * (d * d).sum(axis=-1)).sum())


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64.
    Exact: a bf16 value is an fp64 value with 8 significant bits."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2^e, 0.5 <= |m| < 1
    scaled = m * 256.0                     # 8 significant bits in the integer part
    r = np.round(scaled)                   # numpy rounds half to even
    return np.ldexp(r / 256.0, e)
