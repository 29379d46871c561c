"""Loop-aware codebook fine-tuning (LoopVQ review, arXiv 2611.05304, section
3.2, eq. 6) on top of the compressed-cache attention kernels.

* CompressedAttention -- autograd function: forward is loopvq_prefill_attn
  (causal attention of the positions after the sinks over the cache rebuilt
  from the codebooks), backward is loopvq_prefill_attn_backward (gradients of
  the queries and of the codebook entries; the assignment is a constant, so
  no straight-through estimator is involved).
* ToyLoopedStack -- a synthetic looped model: one attention layer applied at
  every loop step with shared frozen weights (h_{t+1} = h_t + o_t W_o,
  queries RoPE(rmsnorm(h_t) W_q), logits rmsnorm(h_T) W_u).  Real use plugs
  in a model's own layers instead; the kernels do not depend on it.
* finetune_codebooks -- the section 3.2 loop: every iteration re-encodes the
  cache with the current codebooks, runs the stack over the rebuilt cache,
  takes KL(p || q) against the precise run's outputs, backpropagates into the
  codebooks and makes one Adam step on fp32 master copies (the kernels read
  their bf16 rounding).
* PreciseAttention / fisher_importance -- the importance weights of the
  codebook k-means ("codebook and calibration", eq. 3): the stack attends to
  the precise cache (loopvq_precise_attn), the next-token loss against the
  given targets is backpropagated (loopvq_precise_attn_backward adds the
  gradient of every cached key and value), and loopvq_fisher_weights turns
  those gradients into omega_n = ||dL/dz_n||^2 per joint vector.
"""

import torch

from . import api


class _CallState:
    """Per-call constants of CompressedAttention (indices, bf16 codebooks,
    sinks, RoPE table, step)."""

    def __init__(self, g, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, step, pt=None):
        self.g, self.k_idx, self.v_idx = g, k_idx, v_idx
        self.k_cb, self.v_cb = k_cb, v_cb
        self.sink_k, self.sink_v, self.rope, self.step, self.pt = sink_k, sink_v, rope, step, pt


class CompressedAttention(torch.autograd.Function):
    """o = attention(q, rebuilt cache) for one loop step.

    q fp32 [B][Hq][1][N][D] (post-RoPE); k_master / v_master fp32 codebooks
    [H][n_blk][K][G] whose bf16 rounding (st.k_cb / st.v_cb) the kernels read.
    The gradient with respect to those bf16 entries is returned for the fp32
    masters."""

    @staticmethod
    def forward(ctx, q, k_master, v_master, st):
        q = q.contiguous()
        out, lse = api.prefill_attn(st.g, q, st.k_idx, st.v_idx, st.k_cb, st.v_cb, st.sink_k, st.sink_v,
                                    st.rope, step0=st.step, pt=st.pt)
        ctx.save_for_backward(q, out, lse)
        ctx.st = st
        return out

    @staticmethod
    def backward(ctx, d_out):
        q, out, lse = ctx.saved_tensors
        st = ctx.st
        d_q, d_k, d_v = api.prefill_attn_backward(st.g, q, st.k_idx, st.v_idx, st.k_cb, st.v_cb, st.sink_k,
                                                  st.sink_v, st.rope, out, lse, d_out.contiguous(),
                                                  step0=st.step, pt=st.pt)
        return d_q, d_k, d_v, None


def rms_norm(h, eps=1.0e-6):
    return h * torch.rsqrt((h * h).mean(dim=-1, keepdim=True) + eps)


class ToyLoopedStack:
    """Synthetic looped attention stack with frozen weights Wq, Wo [d][d],
    Wu [d][vocab] (d = Hq * D) over T loop steps."""

    def __init__(self, Wq, Wo, Wu, n_q_heads, D, T, n_s, rope):
        self.Wq, self.Wo, self.Wu = Wq, Wo, Wu
        self.Hq, self.D, self.T, self.n_s = n_q_heads, D, T, n_s
        self.rope = rope                      # fp32 [n_pos][D/2][2]

    def _rotate(self, Q):
        """Q [B, Hq, N, D] at positions n_s .. n_s + N - 1."""
        N = Q.shape[2]
        cs = self.rope[self.n_s:self.n_s + N]
        c, s = cs[..., 0], cs[..., 1]
        h = self.D // 2
        a, b = Q[..., :h], Q[..., h:]
        return torch.cat([a * c - b * s, b * c + a * s], dim=-1)

    def logits(self, x, attend):
        """x [B, N, d] -> logits [B, N, vocab]; attend(t, Q [B, Hq, N, D]) -> [B, Hq, N, D]."""
        B, N, d = x.shape
        h = x
        for t in range(self.T):
            Q = (rms_norm(h) @ self.Wq).reshape(B, N, self.Hq, self.D).transpose(1, 2)
            o = attend(t, self._rotate(Q))
            h = h + o.transpose(1, 2).reshape(B, N, d) @ self.Wo
        return rms_norm(h) @ self.Wu


def precise_attend(g, k, v, sink_k, sink_v, rope):
    """attend() over the stored bf16 cache k, v [B][H][T][N][D] (pre-RoPE keys)
    with the bf16 sinks (loopvq_precise_attn): the precise run the codebooks
    are fitted against."""
    def attend(t, Q):
        out, _ = api.precise_attn(g, Q[:, :, None].contiguous(), k, v, sink_k, sink_v, rope, step0=t)
        return out[:, :, 0]
    return attend


def kl_objective(logp, logits_q):
    """Sum over batch entries of mean_j KL(p_j || q_j); logp = log p (fixed)."""
    lq = torch.log_softmax(logits_q, dim=-1)
    return (logp.exp() * (logp - lq)).sum(dim=-1).mean(dim=-1).sum()


def compressed_logits(stack, g, x, k, v, sink_k, sink_v, k_idx, v_idx, k_master, v_master, pt=None):
    """The stack's logits over the cache rebuilt from the (bf16-rounded)
    master codebooks with the given assignment (pt: the keys' pre-transform,
    whose sigma the encode wrote)."""
    kb, vb = k_master.detach().to(torch.bfloat16), v_master.detach().to(torch.bfloat16)

    def attend(t, Q):
        st = _CallState(g, k_idx, v_idx, kb, vb, sink_k, sink_v, stack.rope, t, pt)
        return CompressedAttention.apply(Q[:, :, None], k_master, v_master, st)[:, :, 0]
    return stack.logits(x, attend)


def reassign(g, k, v, k_cb, v_cb, k_idx=None, v_idx=None, pt=None):
    """Exact assignment of the cache to bf16 codebooks (loopvq_encode; with pt
    the keys are coded in the pre-transformed space and sigma is written)."""
    B, H, T, N, D = k.shape
    shp = (B, H, T // g.T_c, N, D // (g.G // g.T_c))
    if k_idx is None:
        k_idx = torch.empty(shp, dtype=torch.uint8, device=k.device)
        v_idx = torch.empty(shp, dtype=torch.uint8, device=k.device)
    api.encode(g, k, k_cb, k_idx, pt=pt)
    api.encode(g, v, v_cb, v_idx)
    return k_idx, v_idx


def finetune_codebooks(stack, g, x, k, v, sink_k, sink_v, k_cb, v_cb, iters, lr=1.0e-3, callback=None, pt=None):
    """Fine-tune bf16 codebooks k_cb, v_cb [H][n_blk][K][G] against the
    stack's precise outputs.  Returns (fp32 masters, list of J before each
    step).  callback(it, J) is called after every iteration."""
    with torch.no_grad():
        logp = torch.log_softmax(stack.logits(x, precise_attend(g, k, v, sink_k, sink_v, stack.rope)), -1)
    km = k_cb.float().clone().requires_grad_(True)
    vm = v_cb.float().clone().requires_grad_(True)
    opt = torch.optim.Adam([km, vm], lr=lr)
    k_idx = v_idx = None
    Js = []
    for it in range(iters):
        k_idx, v_idx = reassign(g, k, v, km.detach().to(torch.bfloat16), vm.detach().to(torch.bfloat16),
                                k_idx, v_idx, pt)
        J = kl_objective(logp, compressed_logits(stack, g, x, k, v, sink_k, sink_v, k_idx, v_idx, km, vm, pt))
        opt.zero_grad(set_to_none=True)
        J.backward()
        opt.step()
        Js.append(float(J.detach()))
        if callback is not None:
            callback(it, Js[-1])
    return km.detach(), vm.detach(), Js


class _PreciseState:
    """Per-call constants of PreciseAttention and the cache-gradient buffers
    its backward adds into."""

    def __init__(self, g, k, v, sink_k, sink_v, rope, step, d_k, d_v):
        self.g, self.k, self.v = g, k, v
        self.sink_k, self.sink_v, self.rope, self.step = sink_k, sink_v, rope, step
        self.d_k, self.d_v = d_k, d_v


class PreciseAttention(torch.autograd.Function):
    """o = attention(q, precise cache) for one loop step.  `anchor` is a
    scalar that requires grad, so that the backward runs even when q does
    not; the backward returns d_q and adds the step's cache gradients into
    st.d_k / st.d_v."""

    @staticmethod
    def forward(ctx, q, anchor, st):
        q = q.contiguous()
        out, lse = api.precise_attn(st.g, q, st.k, st.v, st.sink_k, st.sink_v, st.rope, step0=st.step)
        ctx.save_for_backward(q, out, lse, anchor)
        ctx.st = st
        return out

    @staticmethod
    def backward(ctx, d_out):
        q, out, lse, anchor = ctx.saved_tensors
        st = ctx.st
        d_q = api.precise_attn_backward(st.g, q, st.k, st.v, st.sink_k, st.sink_v, st.rope, out, lse,
                                        d_out.contiguous(), st.d_k, st.d_v, step0=st.step)
        return d_q, torch.zeros_like(anchor), None


def fisher_importance(stack, g, x, k, v, sink_k, sink_v, targets, pt=None):
    """Importance weights of every joint vector of the precise cache k, v
    bf16 [B][H][T][N][D]: L = sum over batch entries of the mean next-token
    cross-entropy of the stack against targets int64 [B][N]; returns
    (L, omega_k, omega_v) with omega fp32 [B][H][n_blk][N][D/c] (pt: the keys'
    pre-transform, whose sigma the encode wrote, to weight key vectors in the
    transformed space)."""
    B, N = targets.shape
    d_k = torch.zeros(k.shape, dtype=torch.float32, device=k.device)
    d_v = torch.zeros(v.shape, dtype=torch.float32, device=v.device)
    anchor = torch.zeros((), dtype=torch.float32, device=k.device, requires_grad=True)

    def attend(t, Q):
        st = _PreciseState(g, k, v, sink_k, sink_v, stack.rope, t, d_k, d_v)
        return PreciseAttention.apply(Q[:, :, None], anchor, st)[:, :, 0]
    with torch.enable_grad():
        logits = stack.logits(x, attend)
        lq = torch.log_softmax(logits, dim=-1)
        L = -lq.gather(-1, targets[..., None]).squeeze(-1).mean(dim=-1).sum()
        L.backward()
    omega_k, omega_v = api.fisher_weights(g, d_k, d_v, N, pt)
    return float(L.detach()), omega_k, omega_v
