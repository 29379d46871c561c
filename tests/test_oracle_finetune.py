"""Pins of the oracle's fine-tuning objective (LoopVQ review, section 3.2,
eq. 6) and of the causal attention over the rebuilt cache: library routines
(scaled_dot_product_attention, scipy's rel_entr and logsumexp, torch.optim's
Adam), closed forms, exact reconstruction and central finite differences."""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as Fnn

import oracle as ref

F64 = torch.float64


def _rng_cache(seed, B=1, H_kv=1, T=4, N=6, D=16, n_s=2):
    g = torch.Generator().manual_seed(seed)
    c = dict(k=torch.randn((B, H_kv, T, N, D), generator=g, dtype=F64),
             v=torch.randn((B, H_kv, T, N, D), generator=g, dtype=F64),
             sink_k=torch.randn((B, H_kv, T, n_s, D), generator=g, dtype=F64),
             sink_v=torch.randn((B, H_kv, T, n_s, D), generator=g, dtype=F64))
    return c, g


def _toy(g, B, N, H_q, D, vocab=7):
    d = H_q * D
    return dict(x=torch.randn((B, N, d), generator=g, dtype=F64),
                Wq=torch.randn((d, d), generator=g, dtype=F64) / math.sqrt(d),
                Wo=torch.randn((d, d), generator=g, dtype=F64) * (0.5 / math.sqrt(d)),
                Wu=torch.randn((d, vocab), generator=g, dtype=F64) * (2.0 / math.sqrt(d)))


def test_causal_attention_matches_sdpa():
    g = torch.Generator().manual_seed(1)
    N, D, n_s = 9, 16, 3
    q = torch.randn((N, D), generator=g, dtype=F64)
    k = torch.randn((N, D), generator=g, dtype=F64)
    v = torch.randn((N, D), generator=g, dtype=F64)
    sk = torch.randn((n_s, D), generator=g, dtype=F64)
    sv = torch.randn((n_s, D), generator=g, dtype=F64)
    o, lse = ref.causal_attention(q, k, v, sk, sv)
    # the same keys rotated by the already pinned numpy RoPE, fed to the library
    keys = np.concatenate([sk.numpy(), k.numpy()])
    kr = torch.from_numpy(ref.apply_rope(keys, np.arange(n_s + N)))
    vals = torch.cat([sv, v])
    mask = torch.zeros((N, n_s + N), dtype=torch.bool)
    for i in range(N):
        mask[i, :n_s + i + 1] = True
    want = Fnn.scaled_dot_product_attention(q[None, None], kr[None, None], vals[None, None],
                                            attn_mask=mask[None, None])[0, 0]
    assert torch.allclose(o, want, rtol=1e-12, atol=1e-12)
    s = (q.numpy() @ kr.numpy().T) / math.sqrt(D)
    for i in range(N):
        assert abs(lse[i].item() - scipy.special.logsumexp(s[i, :n_s + i + 1])) < 1e-12


def test_causal_structure_closed_forms():
    g = torch.Generator().manual_seed(2)
    N, D, n_s = 7, 8, 2
    q = torch.randn((N, D), generator=g, dtype=F64)
    k = torch.randn((N, D), generator=g, dtype=F64)
    v = torch.randn((N, D), generator=g, dtype=F64)
    sk = torch.randn((n_s, D), generator=g, dtype=F64)
    sv = torch.randn((n_s, D), generator=g, dtype=F64)
    o, _ = ref.causal_attention(q, k, v, sk, sv)
    # a later token does not reach an earlier query
    k2, v2 = k.clone(), v.clone()
    k2[5] += 3.0
    v2[5] -= 2.0
    o2, _ = ref.causal_attention(q, k2, v2, sk, sv)
    assert torch.equal(o[:5], o2[:5]) and not torch.allclose(o[5:], o2[5:])
    # q = 0: uniform weights over the sinks and the tokens up to i
    o0, lse0 = ref.causal_attention(torch.zeros_like(q), k, v, sk, sv)
    for i in range(N):
        vals = torch.cat([sv, v[:i + 1]])
        assert torch.allclose(o0[i], vals.mean(dim=0), rtol=1e-13, atol=1e-13)
        assert abs(lse0[i].item() - math.log(n_s + i + 1)) < 1e-13
    # no sinks, one token: the output is that token's value
    o1, lse1 = ref.causal_attention(q[:1], k[:1], v[:1], sk[:0], sv[:0])
    assert torch.equal(o1[0], v[0])
    kr = torch.from_numpy(ref.apply_rope(k[:1].numpy(), np.array([0])))
    assert abs(lse1[0].item() - (q[0] @ kr[0]).item() / math.sqrt(D)) < 1e-13


def test_dequant_step_matches_pinned_dequant():
    rng = np.random.default_rng(3)
    T_c, G, D, N, K = 4, 8, 16, 5, 6
    cb = rng.standard_normal((2, K, G))
    idx = rng.integers(0, K, (2, N, D // (G // T_c)))
    want = ref.dequant(idx, cb, T_c, D)                 # [T, N, D]
    for t in range(8):
        beta, m = divmod(t, T_c)
        got = ref.dequant_step_t(torch.from_numpy(idx[beta]), torch.from_numpy(cb[beta]), T_c, m)
        assert np.array_equal(got.numpy(), want[t])


def test_kl_matches_scipy():
    rng = np.random.default_rng(4)
    a, b = rng.standard_normal((5, 11)), rng.standard_normal((5, 11)) * 2
    got = ref.kl_rows(torch.from_numpy(a), torch.from_numpy(b)).numpy()
    p = scipy.special.softmax(a, axis=1)
    q = scipy.special.softmax(b, axis=1)
    want = scipy.special.rel_entr(p, q).sum(axis=1)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)
    assert np.all(got > 0)
    assert np.allclose(ref.kl_rows(torch.from_numpy(a), torch.from_numpy(a)).numpy(), 0.0, atol=1e-15)


def _codeword_cache(seed, B, H_kv, T, T_c, N, D, n_s, K, G):
    """A cache every token of which is a codeword: the rebuilt cache equals it."""
    rng = np.random.default_rng(seed)
    c = G // T_c
    n_blk = T // T_c
    cb_k = ref.bf16_round(rng.standard_normal((H_kv, n_blk, K, G)))
    cb_v = ref.bf16_round(rng.standard_normal((H_kv, n_blk, K, G)))
    ki = rng.integers(0, K, (B, H_kv, n_blk, N, D // c))
    vi = rng.integers(0, K, (B, H_kv, n_blk, N, D // c))
    k = np.empty((B, H_kv, T, N, D))
    v = np.empty((B, H_kv, T, N, D))
    for b in range(B):
        for h in range(H_kv):
            k[b, h] = ref.dequant(ki[b, h], cb_k[h], T_c, D)
            v[b, h] = ref.dequant(vi[b, h], cb_v[h], T_c, D)
    sink = rng.standard_normal((2, B, H_kv, T, n_s, D))
    cache = dict(k=torch.from_numpy(k), v=torch.from_numpy(v), sink_k=torch.from_numpy(sink[0]),
                 sink_v=torch.from_numpy(sink[1]))
    return cache, torch.from_numpy(cb_k), torch.from_numpy(cb_v), torch.from_numpy(ki), torch.from_numpy(vi)


def test_objective_vanishes_at_exact_reconstruction():
    B, H_kv, H_q, T, T_c, N, D, n_s, K, G = 2, 1, 2, 4, 4, 5, 16, 2, 8, 8
    cache, kc, vc, ki, vi = _codeword_cache(5, B, H_kv, T, T_c, N, D, n_s, K, G)
    cache.update(H_q=H_q, N=N)
    toy = _toy(torch.Generator().manual_seed(6), B, N, H_q, D)
    J, gk, gv = ref.finetune_grad(toy, cache, ki, vi, kc, vc, T_c)
    assert abs(J.item()) < 1e-14
    assert gk.abs().max().item() < 1e-12 and gv.abs().max().item() < 1e-12
    # the exact assignment of such a cache is the generating one (no ties in fp64)
    ki2, vi2 = ref.reassign(cache, kc, vc, T_c)
    assert torch.equal(ki2, ki) and torch.equal(vi2, vi)


def _perturbed_setup(seed, B=1, H_kv=1, H_q=2, T=4, T_c=4, N=5, D=16, n_s=2, K=8, G=8):
    cache, kc, vc, ki, vi = _codeword_cache(seed, B, H_kv, T, T_c, N, D, n_s, K, G)
    g = torch.Generator().manual_seed(seed + 1)
    cache["k"] = cache["k"] + 0.3 * torch.randn(cache["k"].shape, generator=g, dtype=F64)
    cache["v"] = cache["v"] + 0.3 * torch.randn(cache["v"].shape, generator=g, dtype=F64)
    cache.update(H_q=H_q, N=N)
    toy = _toy(g, B, N, H_q, D)
    return toy, cache, kc, vc, ki, vi, T_c


def test_gradient_matches_finite_differences():
    toy, cache, kc, vc, ki, vi, T_c = _perturbed_setup(7)
    J, gk, gv = ref.finetune_grad(toy, cache, ki, vi, kc, vc, T_c)
    assert J.item() > 0
    rng = np.random.default_rng(8)
    used = sorted(set(ki.flatten().tolist()) & set(vi.flatten().tolist()))
    eps = 1e-6
    for which, cb, grad in (("k", kc, gk), ("v", vc, gv)):
        for _ in range(4):
            r = int(rng.choice(used))
            u = int(rng.integers(cb.shape[-1]))
            plus, minus = cb.clone(), cb.clone()
            plus[0, 0, r, u] += eps
            minus[0, 0, r, u] -= eps
            args_p = (plus, vc) if which == "k" else (kc, plus)
            args_m = (minus, vc) if which == "k" else (kc, minus)
            jp = ref.finetune_objective(toy, cache, ki, vi, *args_p, T_c)[0].item()
            jm = ref.finetune_objective(toy, cache, ki, vi, *args_m, T_c)[0].item()
            fd = (jp - jm) / (2 * eps)
            g = grad[0, 0, r, u].item()
            assert abs(fd - g) <= 1e-6 * max(abs(g), 1e-3), (which, r, u, fd, g)
    # a codeword no token uses gets no gradient
    unused = sorted(set(range(kc.shape[2])) - set(ki.flatten().tolist()))
    for r in unused:
        assert torch.count_nonzero(gk[0, 0, r]) == 0


def test_attention_vjp_matches_finite_differences():
    rng = np.random.default_rng(9)
    B, H_kv, H_q, T, T_c, N, D, n_s, K, G = 1, 1, 2, 4, 4, 6, 16, 2, 8, 8
    cache, kc, vc, ki, vi = _codeword_cache(10, B, H_kv, T, T_c, N, D, n_s, K, G)
    q = torch.from_numpy(rng.standard_normal((B, H_q, 2, N, D)))
    dout = torch.from_numpy(rng.standard_normal((B, H_q, 2, N, D)))
    args = (ki, vi, kc, vc, cache["sink_k"], cache["sink_v"], T_c)
    o, lse, dq, dk, dv = ref.attention_vjp(q, *args, dout, step0=1)

    def loss(qq, kk, vv):
        oo, _ = ref.compressed_attention(qq, ki, vi, kk, vv, cache["sink_k"], cache["sink_v"], T_c, 1)
        return float((oo * dout).sum())
    eps = 1e-6
    for _ in range(4):
        pos = tuple(int(rng.integers(s)) for s in q.shape)
        qp, qm = q.clone(), q.clone()
        qp[pos] += eps
        qm[pos] -= eps
        fd = (loss(qp, kc, vc) - loss(qm, kc, vc)) / (2 * eps)
        assert abs(fd - dq[pos].item()) <= 1e-6 * max(abs(dq[pos].item()), 1e-3)
    for which in ("k", "v"):
        grad = dk if which == "k" else dv
        r = int(ki[0, 0, 0, 0, 0]) if which == "k" else int(vi[0, 0, 0, 0, 0])
        for u in range(2):
            cp, cm = (kc if which == "k" else vc).clone(), (kc if which == "k" else vc).clone()
            cp[0, 0, r, u] += eps
            cm[0, 0, r, u] -= eps
            lp = loss(q, cp, vc) if which == "k" else loss(q, kc, cp)
            lm = loss(q, cm, vc) if which == "k" else loss(q, kc, cm)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[0, 0, r, u].item()) <= 1e-6 * max(abs(fd), 1e-3)


def test_adam_matches_torch_optim():
    g = torch.Generator().manual_seed(11)
    p0 = torch.randn(20, generator=g, dtype=F64)
    grads = [torch.randn(20, generator=g, dtype=F64) for _ in range(6)]
    p = p0.clone()
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    tp = torch.nn.Parameter(p0.clone())
    opt = torch.optim.Adam([tp], lr=1e-3)
    for i, gr in enumerate(grads, 1):
        ref.adam_step(p, gr, m, v, i)
        tp.grad = gr.clone()
        opt.step()
    assert torch.allclose(p, tp.detach(), rtol=0, atol=1e-15)


def test_reference_finetuning_lowers_the_objective():
    # direction only: a few Adam iterations from the starting codebooks lower J
    toy, cache, kc, vc, ki, vi, T_c = _perturbed_setup(12, N=6)
    Js, kb, vb = ref.finetune_reference(toy, cache, kc, vc, T_c, iters=12, lr=1e-2)
    assert Js[-1] < Js[0]
    assert np.array_equal(ref.bf16_round(kb.numpy()), kb.numpy())


def test_pretransformed_keys_in_the_attention():
    rng = np.random.default_rng(13)
    D, N, H = 16, 6, 1
    z = rng.standard_normal((N, D))
    w = rng.lognormal(0, 0.3, D)
    perm = rng.permutation(D)
    sig = rng.uniform(0.5, 2, N)
    # the torch inverse equals the pinned numpy inverse, and undoes the forward
    got = ref.tasq_inverse_t(torch.from_numpy(z), w, perm, sig).numpy()
    assert np.allclose(got, ref.tasq_inverse(z, w, perm, sig), rtol=1e-15, atol=0)
    k = rng.standard_normal((N, D))
    back = ref.tasq_inverse_t(torch.from_numpy(ref.tasq_forward(k, w, perm, sig)), w, perm, sig).numpy()
    assert np.allclose(back, k, rtol=1e-14, atol=1e-14)
    # identity transform gives the plain attention exactly
    B, H_q, T, T_c, n_s, K, G = 1, 2, 4, 4, 2, 8, 8
    cache, kc, vc, ki, vi = _codeword_cache(14, B, H, T, T_c, N, D, n_s, K, G)
    q = torch.from_numpy(rng.standard_normal((B, H_q, 2, N, D)))
    args = (q, ki, vi, kc, vc, cache["sink_k"], cache["sink_v"], T_c, 1)
    o0, l0 = ref.compressed_attention(*args)
    ident = (np.ones((H, D)), np.tile(np.arange(D), (H, 1)), np.ones((B, N, T)))
    o1, l1 = ref.compressed_attention(*args, tasq=ident)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    # gradients through the inverse transform match central differences
    tq = (rng.lognormal(0, 0.3, (H, D)), np.stack([rng.permutation(D) for _ in range(H)]),
          rng.uniform(0.5, 2, (B, N, T)))
    dout = torch.from_numpy(rng.standard_normal(q.shape))
    _, _, _, dk, _ = ref.attention_vjp(q, ki, vi, kc, vc, cache["sink_k"], cache["sink_v"], T_c, dout, 1,
                                       tasq=tq)

    def loss(cb):
        o, _ = ref.compressed_attention(q, ki, vi, cb, vc, cache["sink_k"], cache["sink_v"], T_c, 1, tasq=tq)
        return float((o * dout).sum())
    r = int(ki[0, 0, 0, 0, 0])
    for u in range(3):
        cp, cm = kc.clone(), kc.clone()
        cp[0, 0, r, u] += 1e-6
        cm[0, 0, r, u] -= 1e-6
        fd = (loss(cp) - loss(cm)) / 2e-6
        assert abs(fd - dk[0, 0, r, u].item()) <= 1e-6 * max(abs(fd), 1e-3)
