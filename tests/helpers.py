"""Shared helpers for the parity tests: input construction and comparisons.

Inputs come from the seeded generator package; expected values come from the
fp64 oracle.  Nothing here computes a LoopVQ result itself.
"""
import dataclasses
import math

import numpy as np
import torch

import oracle as ref
from synth import build_inputs, config_by_index, random_codebooks  # noqa: F401 (re-exported)

OUT_TOL = 2e-3          # max-abs error relative to the row's output L2 norm


def small_cfg(idx, **over):
    return dataclasses.replace(config_by_index(idx), **over)


def np64(t):
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 or t.dtype == torch.float16 \
        else t.detach().cpu().numpy()


def check_indices(gpu_idx, x, cb, T_c, tasq=None):
    """gpu_idx [n_blk, N, D/c] (numpy), x [T, N, D] fp64, cb [n_blk, K, G] fp64.
    Returns (n_exact, n_tie_ok, n_fail)."""
    if tasq is None:
        want, ties = ref.encode(x, cb, T_c)
        z = ref.joint_vectors(x, T_c, cb.shape[-1])
    else:
        w, perm, sbar = tasq
        want, ties = ref.encode_tasq(x, cb, T_c, w, perm, sbar)
        zt = np.stack([ref.tasq_forward(x[t], w, perm, sbar[:, t]) for t in range(x.shape[0])])
        z = ref.joint_vectors(zt, T_c, cb.shape[-1])
    gi = np.asarray(gpu_idx, dtype=np.int64)
    uniq = ties == 1
    exact = (gi == want)
    n_exact = int((exact & uniq).sum())
    fails = int((~exact & uniq).sum())
    tie_ok = 0
    if (~uniq).any():
        for beta in range(cb.shape[0]):
            m = ~uniq[beta]
            if m.any():
                inset = ref.tie_set_contains(z[beta][m], cb[beta], gi[beta][m])
                tie_ok += int(inset.sum())
                fails += int((~inset).sum())
    return n_exact, tie_ok, fails


def encode_oracle_chunked(gpu_idx, x, cb, T_c, tasq=None, chunk=256):
    tot = [0, 0, 0]
    N = x.shape[1]
    for j0 in range(0, N, chunk):
        j1 = min(N, j0 + chunk)
        t = None if tasq is None else (tasq[0], tasq[1], tasq[2][j0:j1])
        r = check_indices(gpu_idx[:, j0:j1], x[:, j0:j1], cb, T_c, t)
        tot = [a + b for a, b in zip(tot, r)]
    return tuple(tot)


def row_error(o_gpu, o_ref):
    return float(np.max(np.abs(o_gpu - o_ref)) / max(np.linalg.norm(o_ref), 1e-30))
