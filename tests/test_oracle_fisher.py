"""Pins of the oracle's importance weights for the codebook k-means (LoopVQ
review, "codebook and calibration" eq. 3: omega_n = ||dL/dz_n||^2 of joint
vector n, section 3.1: a joint vector covers T_c loop steps): the loss is the
library cross-entropy, each weight equals the sum of squared central finite
differences of the loss along the vector's G coordinates (written from the
joint layout's definition, plain and pre-transformed keys), and frozen
outputs that ignore the cache give zero weights."""
import numpy as np
import pytest
import torch

import oracle as ref

F64 = torch.float64


def _case(seed, B=1, H=2, H_q=2, T=4, N=5, n_s=2, V=16, D=128):
    g = torch.Generator().manual_seed(seed)
    d = H_q * D
    cache = dict(k=torch.randn(B, H, T, N, D, generator=g, dtype=F64),
                 v=torch.randn(B, H, T, N, D, generator=g, dtype=F64),
                 sink_k=torch.randn(B, H, T, n_s, D, generator=g, dtype=F64),
                 sink_v=torch.randn(B, H, T, n_s, D, generator=g, dtype=F64), H_q=H_q, N=N)
    toy = dict(x=torch.randn(B, N, d, generator=g, dtype=F64),
               Wq=torch.randn(d, d, generator=g, dtype=F64) * d ** -0.5,
               Wo=torch.randn(d, d, generator=g, dtype=F64) * (0.5 * d ** -0.5),
               Wu=torch.randn(d, V, generator=g, dtype=F64) * (2.0 * d ** -0.5))
    y = torch.randint(0, V, (B, N), generator=g)
    return toy, cache, y


def test_loss_is_the_library_cross_entropy():
    toy, cache, y = _case(1, B=2)
    L = ref.precise_cache_loss(toy, cache, y)
    want = 0.0
    for b in range(2):
        lg = ref.toy_logits(toy["x"][b], toy["Wq"], toy["Wo"], toy["Wu"], 2, 128, 4, 2,
                            ref._stack_for(b, cache, 1, 1.0e4))
        want += float(torch.nn.functional.cross_entropy(lg, y[b]))
    assert float(L) == pytest.approx(want, rel=1e-13)


def _loss_with(toy, cache, y, key, b, h, t, j, ch, eps):
    c = dict(cache)
    x = cache[key].clone()
    x[b, h, t, j, ch] += eps
    c[key] = x
    return float(ref.precise_cache_loss(toy, c, y))


@pytest.mark.parametrize("T_c,G", [(4, 16), (2, 16), (4, 32)])
def test_weights_are_squared_finite_differences(T_c, G):
    """omega of a joint vector = sum over its coordinates u = i*T_c + m
    (channel q*c + i at block step m) of (dL/dz_u)^2, by central differences."""
    toy, cache, y = _case(2, T=4)
    L, ok, ov = ref.fisher_importance(toy, cache, y.numpy(), T_c, G)
    c = G // T_c
    eps = 1e-5
    for key, om in (("k", ok), ("v", ov)):
        for (b, h, beta, j, q) in [(0, 0, 0, 1, 3), (0, 1, 4 // T_c - 1, 4, 128 // c - 1)]:
            tot = 0.0
            for i in range(c):
                for m in range(T_c):
                    t, ch = beta * T_c + m, q * c + i
                    dlp = _loss_with(toy, cache, y, key, b, h, t, j, ch, eps)
                    dlm = _loss_with(toy, cache, y, key, b, h, t, j, ch, -eps)
                    tot += ((dlp - dlm) / (2 * eps)) ** 2
            assert om[b, h, beta, j, q] == pytest.approx(tot, rel=1e-6, abs=1e-18), (key, b, h, beta, j, q)


def test_pretransformed_key_weights_are_finite_differences_in_the_transformed_space():
    """With z[d'] = w[p(d')] k[p(d')] / sigma, a step along coordinate d' of z
    moves raw channel p(d') of the key by sigma / w[p(d')]."""
    toy, cache, y = _case(3, T=4, N=4)
    rng = np.random.default_rng(3)
    H, D, T, N = 2, 128, 4, 4
    w = rng.lognormal(0.0, 0.3, size=(H, D))
    perm = np.stack([rng.permutation(D) for _ in range(H)])
    sb = rng.uniform(0.5, 2.0, size=(1, N, T))
    L, ok, _ = ref.fisher_importance(toy, cache, y.numpy(), 4, 16, tasq=(w, perm, sb))
    eps = 1e-5
    for (h, j, q) in [(0, 2, 5), (1, 0, 31)]:
        tot = 0.0
        for i in range(4):
            for m in range(4):
                dp = q * 4 + i
                ch = perm[h, dp]
                step = eps * sb[0, j, m] / w[h, ch]
                dlp = _loss_with(toy, cache, y, "k", 0, h, m, j, ch, step)
                dlm = _loss_with(toy, cache, y, "k", 0, h, m, j, ch, -step)
                tot += ((dlp - dlm) / (2 * eps)) ** 2
        assert ok[0, h, 0, j, q] == pytest.approx(tot, rel=1e-6), (h, j, q)


def test_outputs_that_ignore_the_cache_give_zero_weights():
    toy, cache, y = _case(4)
    toy["Wo"] = torch.zeros_like(toy["Wo"])       # attention output never reaches the logits
    L, ok, ov = ref.fisher_importance(toy, cache, y.numpy(), 4, 16)
    assert L > 0 and np.all(ok == 0) and np.all(ov == 0)


def test_weights_cover_the_joint_vector_steps_only():
    """Perturbing a channel at a step outside a block leaves that block's
    vectors' gradient coordinates unchanged: weights of two blocks are made of
    different steps (T = 8, T_c = 4) and both are positive."""
    toy, cache, y = _case(5, T=8, N=4)
    L, ok, ov = ref.fisher_importance(toy, cache, y.numpy(), 4, 16)
    assert ok.shape == (1, 2, 2, 4, 32) and np.all(ok > 0) and np.all(ov > 0)
    # the last query attends every token; the first token is attended by every query,
    # so neither block's weights vanish; T_c = 1 sums per step, and the two
    # groupings add up to the same total
    _, ok1, ov1 = ref.fisher_importance(toy, cache, y.numpy(), 1, 16)
    assert ok1.sum() == pytest.approx(ok.sum(), rel=1e-12) and ov1.sum() == pytest.approx(ov.sum(), rel=1e-12)
