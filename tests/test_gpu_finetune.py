"""GPU parity of the fine-tuning kernels (LoopVQ review, section 3.2, eq. 6)
against the fp64 oracle: the causal attention over the compressed cache, its
backward pass into the queries and the codebook entries, the gradient of the
KL objective through the toy looped stack, and a short fine-tuning run.

Tolerances (fp32 kernels against fp64): outputs, per row, max |err| <= 1e-4 *
||row|| (rows below 1e-3 of the largest use that floor); lse within 1e-4;
gradients, per tensor, max |err| <= 1e-4 * max |ref| (an fp32 sum of n terms
errs by at most ~n * 2^-24 of the sum of magnitudes, and the codebook sums add
up to a few thousand terms).  d_q is checked per row with a floor of 1e-2 of
the largest row: its terms are P (dP - delta) k with dP and delta each rounded
in fp32, so a row's error scales with |dP| |k| however much dP - delta cancels,
and the rows of queries that see one or two keys are small."""
import math

import numpy as np
import pytest
import torch

import oracle as ref
import sub_bit_loop_amd as lv
from sub_bit_loop_amd import finetune as ft
from synth import gen_toy_stack
from tests.helpers import build_inputs, small_cfg

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _setup(cfg, seed=0):
    inp = build_inputs(cfg, 0, "cuda", kmeans=False, cb_seed=3 + seed)
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    shp = (cfg.B, cfg.H_kv, cfg.n_blk, cfg.N + 5, cfg.chunks)   # N_cap > N
    kidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    lv.encode(g, inp["k"], inp["k_cb"], kidx)
    lv.encode(g, inp["v"], inp["v_cb"], vidx)
    rope = lv.rope_table_f32(cfg.n_s + cfg.N + 3, cfg.D, cfg.theta)
    return g, inp, kidx, vidx, rope


def _oracle_args(cfg, inp, kidx, vidx):
    return (kidx.long().cpu(), vidx.long().cpu(), inp["k_cb"].double().cpu(), inp["v_cb"].double().cpu(),
            inp["sink_k"].double().cpu(), inp["sink_v"].double().cpu(), cfg.T_c)


def _row_check(got, want, tol, what, floor=1e-3):
    g = got.double().cpu().reshape(-1, got.shape[-1])
    w = want.reshape(-1, want.shape[-1])
    err = (g - w).abs().max(dim=1).values
    # rows far below the largest (query 0 with no sinks has d_q = 0 exactly)
    # are measured against `floor` times the largest row
    norms = w.norm(dim=1)
    scale = norms.clamp_min(floor * float(norms.max()))
    worst = float((err / scale).max())
    _say("  %s worst rel err %.3g (tolerance %g)" % (what, worst, tol))
    assert worst <= tol, what
    return worst


def _tensor_check(got, want, tol, what):
    g = got.double().cpu()
    scale = float(want.abs().max())
    err = float((g - want).abs().max())
    _say("  %s max err %.3g of max %.3g (tolerance %g)" % (what, err, scale, tol))
    assert err <= tol * scale, what


GEOMS = [
    # name, G, T_c, T, H_kv, H_q, B, N, n_s, step0, n_steps
    ("c4-gqa2", 16, 4, 4, 2, 4, 2, 150, 4, 1, 3),
    ("c8-2blk", 16, 2, 4, 1, 2, 1, 97, 4, 0, 4),
    ("c8-g32", 32, 4, 4, 1, 1, 1, 130, 0, 0, 4),
    ("c16-tc1", 16, 1, 2, 1, 1, 2, 65, 3, 1, 1),
]


@pytest.mark.parametrize("name,G,T_c,T,H_kv,H_q,B,N,n_s,step0,n_steps", GEOMS)
def test_prefill_forward_backward(name, G, T_c, T, H_kv, H_q, B, N, n_s, step0, n_steps):
    _say("prefill attention %s" % name)
    cfg = small_cfg(1, G=G, T_c=T_c, T=T, H_kv=H_kv, H_q=H_q, B=B, N=N, n_s=max(n_s, 1),
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1))
    g, inp, kidx, vidx, rope = _setup(cfg)
    gq = torch.Generator(device="cpu").manual_seed(11)
    q = torch.randn((B, H_q, n_steps, N, cfg.D), generator=gq).cuda()
    dout = torch.randn((B, H_q, n_steps, N, cfg.D), generator=gq).cuda()
    sk = inp["sink_k"][:, :, :, :n_s].contiguous() if n_s else None
    sv = inp["sink_v"][:, :, :, :n_s].contiguous() if n_s else None
    out, lse = lv.prefill_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, step0=step0)
    dq, dk, dv = lv.prefill_attn_backward(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, out, lse,
                                          dout, step0=step0)
    torch.cuda.synchronize()
    ka, va, kc, vc, sks, svs, _ = _oracle_args(cfg, inp, kidx, vidx)
    sks, svs = sks[:, :, :, :n_s], svs[:, :, :, :n_s]
    o_r, l_r, dq_r, dk_r, dv_r = ref.attention_vjp(q.double().cpu(), ka, va, kc, vc, sks, svs, T_c,
                                                   dout.double().cpu(), step0=step0, theta=cfg.theta)
    _row_check(out, o_r, 1e-4, "out")
    dl = float((lse.double().cpu() - l_r).abs().max())
    _say("  lse max err %.3g" % dl)
    assert dl <= 1e-4
    _row_check(dq, dq_r, 1e-4, "d_q", floor=1e-2)
    _tensor_check(dk, dk_r, 1e-4, "d_k_cb")
    _tensor_check(dv, dv_r, 1e-4, "d_v_cb")
    # the forward is deterministic
    out2, lse2 = lv.prefill_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, step0=step0)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_prefill_empty_and_unused_codewords():
    cfg = small_cfg(1, N=40, B=1, n_s=2)
    g, inp, kidx, vidx, rope = _setup(cfg)
    q = torch.zeros((1, 1, 4, 0, cfg.D), device="cuda")
    dk = torch.full(inp["k_cb"].shape, 7.0, device="cuda")
    dv = torch.full(inp["v_cb"].shape, 7.0, device="cuda")
    out, lse = lv.prefill_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"], rope)
    lv.prefill_attn_backward(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"], rope,
                             out, lse, torch.zeros_like(q), d_k_cb=dk, d_v_cb=dv)
    torch.cuda.synchronize()
    assert out.numel() == 0 and int(torch.count_nonzero(dk)) == 0 and int(torch.count_nonzero(dv)) == 0
    # codewords no token uses get exactly zero gradient
    q = torch.randn((1, 1, 4, cfg.N, cfg.D), device="cuda")
    out, lse = lv.prefill_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"], rope)
    _, dk, dv = lv.prefill_attn_backward(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"],
                                         inp["sink_v"], rope, out, lse, torch.randn_like(q))
    torch.cuda.synchronize()
    used = set(kidx[0, 0, 0, :cfg.N].flatten().tolist())
    unused = [r for r in range(cfg.K) if r not in used]
    assert unused and int(torch.count_nonzero(dk[0, 0, unused])) == 0


def _toy_case(N=72, vocab=64, B=2):
    cfg = small_cfg(1, T=4, T_c=4, G=16, H_kv=1, H_q=2, B=B, N=N, n_s=4)
    g, inp, kidx, vidx, rope = _setup(cfg)
    toy = gen_toy_stack(cfg, 0, "cuda", vocab=vocab)
    stack = ft.ToyLoopedStack(toy["Wq"], toy["Wo"], toy["Wu"], cfg.H_q, cfg.D, cfg.T, cfg.n_s, rope)
    return cfg, g, inp, kidx, vidx, rope, toy, stack


def test_finetune_gradient_matches_oracle():
    _say("fine-tuning objective and codebook gradient through the toy stack")
    cfg, g, inp, kidx, vidx, rope, toy, stack = _toy_case()
    kidx = kidx[:, :, :, :cfg.N].contiguous()
    vidx = vidx[:, :, :, :cfg.N].contiguous()
    with torch.no_grad():
        logp = torch.log_softmax(stack.logits(toy["x"], ft.precise_attend(g, inp["k"], inp["v"], inp["sink_k"],
                                                                            inp["sink_v"], rope)), -1)
    km = inp["k_cb"].float().clone().requires_grad_(True)
    vm = inp["v_cb"].float().clone().requires_grad_(True)
    J = ft.kl_objective(logp, ft.compressed_logits(stack, g, toy["x"], inp["k"], inp["v"], inp["sink_k"],
                                                   inp["sink_v"], kidx, vidx, km, vm))
    J.backward()
    torch.cuda.synchronize()
    t64, c64 = ref.to_f64_inputs(toy, inp, cfg.H_q, cfg.N)
    J_r, gk_r, gv_r = ref.finetune_grad(t64, c64, kidx.long().cpu(), vidx.long().cpu(),
                                        inp["k_cb"].double().cpu(), inp["v_cb"].double().cpu(), cfg.T_c, cfg.theta)
    rel = abs(float(J) - float(J_r)) / float(J_r)
    _say("  J gpu %.6g oracle %.6g rel %.3g" % (float(J), float(J_r), rel))
    assert rel <= 1e-3
    _tensor_check(km.grad, gk_r, 2e-3, "dJ/dk_cb")
    _tensor_check(vm.grad, gv_r, 2e-3, "dJ/dv_cb")


def test_finetune_loop_lowers_objective():
    _say("fine-tuning loop (Adam, re-encode every iteration)")
    cfg, g, inp, kidx, vidx, rope, toy, stack = _toy_case(N=96)
    km, vm, Js = ft.finetune_codebooks(stack, g, toy["x"], inp["k"], inp["v"], inp["sink_k"], inp["sink_v"],
                                       inp["k_cb"], inp["v_cb"], iters=12, lr=1e-2)
    _say("  J: %s" % " ".join("%.4g" % j for j in Js))
    assert all(math.isfinite(j) for j in Js)
    assert Js[-1] < Js[0]


def test_prefill_full_size_sampled():
    # the fine-tuning workload bench.py times (16 kv-heads / 16 q-heads, 2048
    # tokens + 4 sinks, 4 steps in one call); the oracle recomputes two q-heads
    # (every step and query) and, since MHA gives each kv-head one q-head, the
    # complete codebook gradients of kv-head 5
    from dataclasses import replace
    from synth import config_by_index
    cfg = replace(config_by_index(2), B=1, N=2048)
    _say("prefill attention at full size: B=1 H=16 N=2048 T=4")
    g, inp, kidx, vidx, rope = _setup(cfg)
    gq = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn((1, cfg.H_q, cfg.T, cfg.N, cfg.D), generator=gq, device="cuda")
    dout = torch.randn((1, cfg.H_q, cfg.T, cfg.N, cfg.D), generator=gq, device="cuda")
    out, lse = lv.prefill_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"], rope)
    dq, dk, dv = lv.prefill_attn_backward(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"],
                                          inp["sink_v"], rope, out, lse, dout)
    torch.cuda.synchronize()
    for h in (5, 15):
        sl = slice(h, h + 1)
        o_r, l_r, dq_r, dk_r, dv_r = ref.attention_vjp(
            q[:, sl].double().cpu(), kidx[:, sl, :, :cfg.N].long().cpu(), vidx[:, sl, :, :cfg.N].long().cpu(),
            inp["k_cb"][sl].double().cpu(), inp["v_cb"][sl].double().cpu(), inp["sink_k"][:, sl].double().cpu(),
            inp["sink_v"][:, sl].double().cpu(), cfg.T_c, dout[:, sl].double().cpu(), theta=cfg.theta)
        _row_check(out[:, sl], o_r, 1e-4, "out head %d" % h)
        dl = float((lse[:, sl].double().cpu() - l_r).abs().max())
        _say("  lse head %d max err %.3g" % (h, dl))
        assert dl <= 1e-4
        _row_check(dq[:, sl], dq_r, 1e-4, "d_q head %d" % h, floor=1e-2)
        if h == 5:
            _tensor_check(dk[sl], dk_r, 1e-4, "d_k_cb kv-head 5")
            _tensor_check(dv[sl], dv_r, 1e-4, "d_v_cb kv-head 5")


@pytest.mark.parametrize("G,H_kv,H_q,N,n_s", [(16, 2, 4, 150, 4), (32, 1, 1, 97, 0)])
def test_prefill_pretransformed_keys(G, H_kv, H_q, N, n_s):
    # keys coded in the pre-transformed space (w, perm per kv-head; sigma per
    # token and step, written by the encode): the kernels rebuild the raw keys
    # and pass the gradient back through the inverse transform
    _say("prefill attention with pre-transformed keys G=%d H=%d/%d N=%d" % (G, H_kv, H_q, N))
    cfg = small_cfg(1, G=G, H_kv=H_kv, H_q=H_q, B=2, N=N, n_s=max(n_s, 1), tasq=True)
    inp = build_inputs(cfg, 0, "cuda", kmeans=False, cb_seed=5)
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    shp = (cfg.B, cfg.H_kv, cfg.n_blk, cfg.N, cfg.chunks)
    kidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    sigma = torch.zeros((cfg.B, cfg.N, cfg.T), dtype=torch.float16, device="cuda")
    pt = lv.pretransform(inp["w"], inp["perm"], sigma)
    lv.encode(g, inp["k"], inp["k_cb"], kidx, pt=pt)
    lv.encode(g, inp["v"], inp["v_cb"], vidx)
    rope = lv.rope_table_f32(cfg.n_s + cfg.N, cfg.D, cfg.theta)
    gq = torch.Generator(device="cpu").manual_seed(21)
    q = torch.randn((cfg.B, H_q, cfg.T, N, cfg.D), generator=gq).cuda()
    dout = torch.randn((cfg.B, H_q, cfg.T, N, cfg.D), generator=gq).cuda()
    sk = inp["sink_k"][:, :, :, :n_s].contiguous() if n_s else None
    sv = inp["sink_v"][:, :, :, :n_s].contiguous() if n_s else None
    out, lse = lv.prefill_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, pt=pt)
    dq, dk, dv = lv.prefill_attn_backward(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, out, lse,
                                          dout, pt=pt)
    torch.cuda.synchronize()
    tq = (inp["w"].double().cpu(), inp["perm"].long().cpu() & (cfg.D - 1), sigma.double().cpu())
    o_r, l_r, dq_r, dk_r, dv_r = ref.attention_vjp(
        q.double().cpu(), kidx.long().cpu(), vidx.long().cpu(), inp["k_cb"].double().cpu(),
        inp["v_cb"].double().cpu(), inp["sink_k"][:, :, :, :n_s].double().cpu(),
        inp["sink_v"][:, :, :, :n_s].double().cpu(), cfg.T_c, dout.double().cpu(), theta=cfg.theta, tasq=tq)
    _row_check(out, o_r, 1e-4, "out")
    dl = float((lse.double().cpu() - l_r).abs().max())
    _say("  lse max err %.3g" % dl)
    assert dl <= 1e-4
    _row_check(dq, dq_r, 1e-4, "d_q", floor=1e-2)
    _tensor_check(dk, dk_r, 1e-4, "d_k_cb")
    _tensor_check(dv, dv_r, 1e-4, "d_v_cb")
