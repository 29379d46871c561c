"""Plain fp64 definition of the loop-aware codebook fine-tuning (eq. 6) on a
toy looped attention stack: causal attention of every position after the
sinks over the cache rebuilt from the codebooks, the KL objective, and its
exact gradient with respect to the codebook entries.

TEST INFRASTRUCTURE: imported only by tests, smoke() and the benchmark's
CPU-baseline leg.

Source: the LoopVQ review page (jaehun.me, "paper-2611-05304v1"):
  * section 3.2 (loop-aware codebook fine-tuning, eq. 6): with the model
    weights frozen, J(B) is the mean over the N positions after the bf16 sink
    tokens of KL(p_j || q_j(B)), where p_j is the output distribution with
    the precise cache and q_j(B) the output when every one of the T_c steps
    attends to the cache rebuilt from the codebooks;
  * same section: the codebook entries receive exact gradients by
    backpropagation because the argmin choice itself is not differentiated
    (no straight-through estimator); the assignment is recomputed with the
    current codebook at every iteration; Adam with learning rate 1e-3, one
    sequence per iteration;
  * section 3.1: RoPE after dequant, step m reads coordinate i*T_c + m of
    the shared codeword.

Readings taken where the pages give no model (listed with their reasons in
the design notes of the repository):
  * the toy stack is one attention layer looped over the T steps with shared
    weights: h_0 = x; at step t the queries are RoPE(rmsnorm(h_t) W_q),
    head-major, at positions n_s + i; o_t is causal attention over step t's
    cache (sinks at 0..n_s-1, token j at n_s + j, attended when j <= i);
    h_{t+1} = h_t + o_t W_o; logits = rmsnorm(h_T) W_u;
  * the cache is an input (the synthetic loop-correlated K/V), not the toy's
    own projections; the precise run reads it as stored (bf16 values), the
    quantized run reads the tokens rebuilt from the codebooks; sinks stay
    bf16 in both;
  * the gradient is taken with respect to the codebook values the forward
    reads (the bf16 entries); an optimizer keeps its own fp32 master copy;
  * the importance weights of the codebook k-means ("codebook and
    calibration", eq. 3: omega_n = ||dL/dz_n||^2) take L as the next-token
    cross-entropy of the toy stack over the precise cache against seeded
    target tokens (no data exists), summed over the batch entries of the
    mean over each sequence's N positions; z_n is a joint vector of the
    precise cache (section 3.1), for pre-transformed keys in the transformed
    space with sigma held at its stored value.
"""
import math

import numpy as np
import torch

F64 = torch.float64


def rope_t(x: torch.Tensor, positions: torch.Tensor, theta: float = 1.0e4) -> torch.Tensor:
    """Rotate-half RoPE on pairs (d, d + D/2) with angle pos * theta^(-2d/D),
    in fp64.  x [..., P, D], positions [P]."""
    D = x.shape[-1]
    h = D // 2
    f = torch.arange(h, dtype=F64)
    omega = torch.pow(torch.tensor(float(theta), dtype=F64), -2.0 * f / D)
    phi = positions.to(F64)[:, None] * omega[None, :]
    c, s = torch.cos(phi), torch.sin(phi)
    a, b = x[..., :h], x[..., h:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def dequant_step_t(idx: torch.Tensor, cb: torch.Tensor, T_c: int, m: int) -> torch.Tensor:
    """Step m of one block (eq. 5): x[j, q*c + i] = cb[idx[j, q], i*T_c + m].
    idx [N, D/c] (int64), cb [K, G] -> [N, D]; differentiable in cb."""
    e = cb[idx]                                   # [N, D/c, G]
    return e[:, :, m::T_c].reshape(idx.shape[0], -1)


def tasq_inverse_t(z: torch.Tensor, w, perm, sigma_bar) -> torch.Tensor:
    """Keys from the pre-transformed space (section 3.3, appendix B eq. 10):
    k[..., p(d')] = z[..., d'] * sigma_bar / w[p(d')], differentiable in z.
    z [..., P, D], w [D], perm [D] (transformed channel d' holds raw channel
    perm[d']), sigma_bar [P]."""
    p = torch.as_tensor(perm, dtype=torch.int64)
    pinv = torch.argsort(p)
    wv = torch.as_tensor(w, dtype=F64)
    sg = torch.as_tensor(sigma_bar, dtype=F64)
    return z[..., pinv] * sg[..., :, None] / wv[None, :]


def causal_attention(q, k_tok, v_tok, sink_k, sink_v, theta: float = 1.0e4):
    """Attention of the N positions after the sinks over one step's cache.

    q [N, D]: post-RoPE queries, query i at position n_s + i.
    k_tok, v_tok [N, D]: pre-RoPE keys / values of token j at n_s + j.
    sink_k, sink_v [n_s, D]: pre-RoPE sinks at positions 0..n_s-1.
    Query i attends to every sink and to tokens j <= i; scale 1/sqrt(D).
    Returns (o [N, D], lse [N]) with the natural log-sum-exp of the scores.
    """
    N, D = q.shape
    n_s = sink_k.shape[0]
    keys = torch.cat([sink_k, k_tok], dim=0)
    vals = torch.cat([sink_v, v_tok], dim=0)
    kr = rope_t(keys, torch.arange(n_s + N), theta)
    s = (q @ kr.T) / math.sqrt(D)
    allowed = torch.ones((N, n_s + N), dtype=torch.bool)
    allowed[:, n_s:] = torch.tril(torch.ones((N, N), dtype=torch.bool))
    s = s.masked_fill(~allowed, float("-inf"))
    lse = torch.logsumexp(s, dim=1)
    o = torch.exp(s - lse[:, None]) @ vals
    return o, lse


def compressed_attention(q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, T_c: int,
                         step0: int = 0, theta: float = 1.0e4, tasq=None):
    """All rows of the causal attention over the compressed cache.

    q [B, H_q, n_steps, N, D] (steps step0 ..), k_idx / v_idx [B, H_kv, n_blk,
    N, D/c] (int64), k_cb / v_cb [H_kv, n_blk, K, G], sink_k / sink_v
    [B, H_kv, T, n_s, D].  tasq: None or (w [H_kv, D], perm [H_kv, D],
    sigma_bar [B, N, T]) for keys coded in the pre-transformed space.
    Returns (o [B, H_q, n_steps, N, D], lse [B, H_q, n_steps, N]);
    differentiable in q, k_cb and v_cb.
    """
    B, H_q, n_steps, N, D = q.shape
    H_kv = k_cb.shape[0]
    gqa = H_q // H_kv
    outs, lses = [], []
    for b in range(B):
        ob, lb = [], []
        for hq in range(H_q):
            h = hq // gqa
            oh, lh = [], []
            for tl in range(n_steps):
                t = step0 + tl
                beta, m = divmod(t, T_c)
                kq = dequant_step_t(k_idx[b, h, beta, :N], k_cb[h, beta], T_c, m)
                if tasq is not None:
                    kq = tasq_inverse_t(kq, tasq[0][h], tasq[1][h], tasq[2][b, :N, t])
                vq = dequant_step_t(v_idx[b, h, beta, :N], v_cb[h, beta], T_c, m)
                o, l = causal_attention(q[b, hq, tl], kq, vq, sink_k[b, h, t], sink_v[b, h, t], theta)
                oh.append(o)
                lh.append(l)
            ob.append(torch.stack(oh))
            lb.append(torch.stack(lh))
        outs.append(torch.stack(ob))
        lses.append(torch.stack(lb))
    return torch.stack(outs), torch.stack(lses)


def attention_vjp(q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, T_c: int, d_out,
                  step0: int = 0, theta: float = 1.0e4, tasq=None):
    """Gradients of <d_out, o> with respect to q, k_cb and v_cb (backprop
    through dequant, RoPE and the softmax; the indices are constants).
    Returns (o, lse, d_q, d_k_cb, d_v_cb) in fp64."""
    qv = torch.as_tensor(q, dtype=F64).clone().requires_grad_(True)
    kc = torch.as_tensor(k_cb, dtype=F64).clone().requires_grad_(True)
    vc = torch.as_tensor(v_cb, dtype=F64).clone().requires_grad_(True)
    o, lse = compressed_attention(qv, k_idx, v_idx, kc, vc, torch.as_tensor(sink_k, dtype=F64),
                                  torch.as_tensor(sink_v, dtype=F64), T_c, step0, theta, tasq)
    (o * torch.as_tensor(d_out, dtype=F64)).sum().backward()
    return o.detach(), lse.detach(), qv.grad, kc.grad, vc.grad


# ----------------------------------------------------------------------------
# toy looped stack and the objective (eq. 6)
# ----------------------------------------------------------------------------

def rms_norm(h: torch.Tensor, eps: float = 1.0e-6) -> torch.Tensor:
    return h / torch.sqrt((h * h).mean(dim=-1, keepdim=True) + eps)


def toy_logits(x, Wq, Wo, Wu, H_q: int, D: int, T: int, n_s: int, attend, theta: float = 1.0e4):
    """x [N, H_q*D] -> logits [N, vocab].  attend(t, Q [H_q, N, D]) returns
    step t's attention output [H_q, N, D] for post-RoPE queries Q."""
    N = x.shape[0]
    pos = n_s + torch.arange(N)
    h = x
    for t in range(T):
        Q = (rms_norm(h) @ Wq).reshape(N, H_q, D).transpose(0, 1)
        o = attend(t, rope_t(Q, pos, theta))
        h = h + o.transpose(0, 1).reshape(N, H_q * D) @ Wo
    return rms_norm(h) @ Wu


def kl_rows(logits_p: torch.Tensor, logits_q: torch.Tensor) -> torch.Tensor:
    """KL(p_j || q_j) per row, natural log."""
    lp = torch.log_softmax(logits_p, dim=-1)
    lq = torch.log_softmax(logits_q, dim=-1)
    return (lp.exp() * (lp - lq)).sum(dim=-1)


def _stack_for(b, inp, T_c, theta, k_cb=None, v_cb=None, k_idx=None, v_idx=None):
    """attend() of batch entry b over the precise cache (k_cb None) or the
    compressed one."""
    x = inp
    H_kv = x["k"].shape[1]
    H_q = x["H_q"]
    gqa = H_q // H_kv
    N = x["N"]

    def attend(t, Q):
        beta, m = divmod(t, T_c)
        outs = []
        for hq in range(H_q):
            h = hq // gqa
            if k_cb is None:
                kq = x["k"][b, h, t, :N]
                vq = x["v"][b, h, t, :N]
            else:
                kq = dequant_step_t(k_idx[b, h, beta, :N], k_cb[h, beta], T_c, m)
                vq = dequant_step_t(v_idx[b, h, beta, :N], v_cb[h, beta], T_c, m)
            o, _ = causal_attention(Q[hq], kq, vq, x["sink_k"][b, h, t], x["sink_v"][b, h, t], theta)
            outs.append(o)
        return torch.stack(outs)
    return attend


def finetune_objective(toy, cache, k_idx, v_idx, k_cb, v_cb, T_c: int, theta: float = 1.0e4):
    """J(B) of eq. (6) summed over the batch entries (each entry one sequence,
    mean over its N positions).

    toy: dict x [B, N, d], Wq, Wo, Wu.  cache: dict k, v [B, H_kv, T, N, D],
    sink_k, sink_v [B, H_kv, T, n_s, D] (bf16 values), H_q.  k_idx / v_idx
    [B, H_kv, n_blk, N, D/c] int64; k_cb / v_cb [H_kv, n_blk, K, G] fp64.
    Returns (J, per-entry J list)."""
    T = cache["k"].shape[2]
    n_s = cache["sink_k"].shape[3]
    D = cache["k"].shape[-1]
    H_q = cache["H_q"]
    per = []
    for b in range(toy["x"].shape[0]):
        args = (toy["x"][b], toy["Wq"], toy["Wo"], toy["Wu"], H_q, D, T, n_s)
        lp = toy_logits(*args, _stack_for(b, cache, T_c, theta), theta)
        lq = toy_logits(*args, _stack_for(b, cache, T_c, theta, k_cb, v_cb, k_idx, v_idx), theta)
        per.append(kl_rows(lp.detach(), lq).mean())
    J = torch.stack(per).sum()
    return J, per


def to_f64_inputs(toy, inp, H_q: int, N: int):
    """fp64 CPU copies of the toy weights and of the cache tensors."""
    c = {k: torch.as_tensor(inp[k]).to("cpu", F64) for k in ("k", "v", "sink_k", "sink_v")}
    c["H_q"] = H_q
    c["N"] = N
    t = {k: torch.as_tensor(v).to("cpu", F64) for k, v in toy.items()}
    return t, c


def finetune_grad(toy, cache, k_idx, v_idx, k_cb, v_cb, T_c: int, theta: float = 1.0e4):
    """(J, dJ/dk_cb, dJ/dv_cb) in fp64 by backpropagation through the toy
    stack, the causal attention, RoPE and the dequant gather."""
    kc = torch.as_tensor(k_cb, dtype=F64).clone().requires_grad_(True)
    vc = torch.as_tensor(v_cb, dtype=F64).clone().requires_grad_(True)
    J, _ = finetune_objective(toy, cache, k_idx, v_idx, kc, vc, T_c, theta)
    J.backward()
    return J.detach(), kc.grad, vc.grad


def adam_step(p, g, m, v, step: int, lr: float = 1.0e-3, b1: float = 0.9, b2: float = 0.999,
              eps: float = 1.0e-8):
    """One Adam update (Kingma and Ba, "Adam: a method for stochastic
    optimization", algorithm 1), in place on fp64 tensors; step >= 1."""
    m.mul_(b1).add_((1.0 - b1) * g)
    v.mul_(b2).add_((1.0 - b2) * g * g)
    mh = m / (1.0 - b1 ** step)
    vh = v / (1.0 - b2 ** step)
    p.sub_(lr * mh / (vh.sqrt() + eps))


def reassign(cache, k_cb, v_cb, T_c: int):
    """Exact assignment of every cached token to the current codebooks
    (eq. 2 over the loop-axis joint vectors); int64 [B, H_kv, n_blk, N, D/c]."""
    from .loopvq_ref import encode
    k = cache["k"].numpy()
    v = cache["v"].numpy()
    B, H = k.shape[:2]
    ki = np.stack([np.stack([encode(k[b, h], k_cb[h].numpy(), T_c)[0] for h in range(H)]) for b in range(B)])
    vi = np.stack([np.stack([encode(v[b, h], v_cb[h].numpy(), T_c)[0] for h in range(H)]) for b in range(B)])
    return torch.from_numpy(ki), torch.from_numpy(vi)


def finetune_reference(toy, cache, k_cb0, v_cb0, T_c: int, iters: int, lr: float = 1.0e-3,
                       theta: float = 1.0e4):
    """The fine-tuning loop of section 3.2 on one batch: every iteration
    re-encodes the cache with the current codebooks rounded to bf16, takes
    the exact gradient of J with respect to those entries and makes one Adam
    step on the fp64 master copy.  Returns (J per iteration, final bf16
    codebooks as fp64)."""
    from .kmeans_ref import bf16_round
    kp = torch.as_tensor(k_cb0, dtype=F64).clone()
    vp = torch.as_tensor(v_cb0, dtype=F64).clone()
    st = [torch.zeros_like(kp), torch.zeros_like(kp), torch.zeros_like(vp), torch.zeros_like(vp)]
    Js = []
    for it in range(1, iters + 1):
        kb = torch.from_numpy(bf16_round(kp.numpy()))
        vb = torch.from_numpy(bf16_round(vp.numpy()))
        ki, vi = reassign(cache, kb, vb, T_c)
        J, gk, gv = finetune_grad(toy, cache, ki, vi, kb, vb, T_c, theta)
        Js.append(float(J))
        adam_step(kp, gk, st[0], st[1], it, lr)
        adam_step(vp, gv, st[2], st[3], it, lr)
    return Js, torch.from_numpy(bf16_round(kp.numpy())), torch.from_numpy(bf16_round(vp.numpy()))


# ----------------------------------------------------------------------------
# importance weights of the codebook k-means (eq. 3) on the toy stack
# ----------------------------------------------------------------------------

def next_token_loss(logits: torch.Tensor, targets: torch.Tensor) -> torch.Tensor:
    """Mean over the rows of -log softmax(logits)[target] (natural log)."""
    lq = torch.log_softmax(logits, dim=-1)
    return -lq.gather(-1, targets[:, None]).mean()


def precise_cache_loss(toy, cache, targets, theta: float = 1.0e4):
    """L = sum over batch entries of the mean next-token loss of the toy stack
    attending to the precise cache (cache["k"], cache["v"] may require grad)."""
    T = cache["k"].shape[2]
    n_s = cache["sink_k"].shape[3]
    D = cache["k"].shape[-1]
    H_q = cache["H_q"]
    L = 0.0
    for b in range(toy["x"].shape[0]):
        lg = toy_logits(toy["x"][b], toy["Wq"], toy["Wo"], toy["Wu"], H_q, D, T, n_s,
                        _stack_for(b, cache, 1, theta), theta)
        L = L + next_token_loss(lg, torch.as_tensor(targets[b], dtype=torch.int64))
    return L


def fisher_importance(toy, cache, targets, T_c: int, G: int, theta: float = 1.0e4, tasq=None):
    """(L, omega_k, omega_v): eq. 3's weight of every joint vector of the
    precise cache, omega = ||dL/dz||^2 over its G coordinates, with
    omega_* [B, H_kv, n_blk, N, D/c] (numpy fp64).

    The gradient with respect to the cached keys and values comes from
    autograd; z is a coordinate permutation of them (section 3.1), and for
    pre-transformed keys (tasq = (w [H_kv, D], perm [H_kv, D], sigma_bar
    [B, N, T])) z[d'] = w[p(d')] k[p(d')] / sigma_bar, so dL/dz[d'] =
    dL/dk[p(d')] sigma_bar / w[p(d')]."""
    from .kmeans_ref import fisher_weights
    from .loopvq_ref import joint_vectors
    N = cache["N"]
    c = dict(cache)
    k = torch.as_tensor(cache["k"][:, :, :, :N], dtype=F64).clone().requires_grad_(True)
    v = torch.as_tensor(cache["v"][:, :, :, :N], dtype=F64).clone().requires_grad_(True)
    c["k"], c["v"] = k, v
    L = precise_cache_loss(toy, c, targets, theta)
    L.backward()
    gk = k.grad.numpy()
    gv = v.grad.numpy()
    if tasq is not None:
        w, perm, sb = (np.asarray(x, dtype=np.float64) for x in tasq)
        perm = perm.astype(np.int64)
        gz = np.empty_like(gk)
        for h in range(gk.shape[1]):
            p = perm[h]
            # [B, T, N, D'] = dL/dk[..., p(d')] * sigma_bar[b, j, t] / w[p(d')]
            gz[:, h] = gk[:, h][..., p] * np.transpose(sb, (0, 2, 1))[:, :, :, None] / w[h][p]
        gk = gz
    ok = fisher_weights(joint_vectors(gk, T_c, G))
    ov = fisher_weights(joint_vectors(gv, T_c, G))
    return float(L.detach()), ok, ov
