"""GPU parity of the importance weights of the codebook k-means (LoopVQ
review, "codebook and calibration" eq. 3: omega_n = ||dL/dz_n||^2; section
3.1: a joint vector covers T_c loop steps) against the fp64 oracle: the
causal attention over the precise cache and its gradients with respect to
the queries and to every cached key and value, the weights of the toy looped
stack's next-token loss (plain and pre-transformed keys), and one weighted
k-means update fed with them.

Tolerances (fp32 kernels against fp64): attention outputs and d_q per row as
in the compressed-cache tests; cache gradients per tensor, max |err| <= 1e-4 *
max |ref|; weights max |err| <= 2e-3 * max |ref| (squares of fp32 gradients
through four loop steps of an fp32 stack)."""
import numpy as np
import pytest
import torch

import oracle as ref
import sub_bit_loop_amd as lv
from sub_bit_loop_amd import finetune as ft
from synth import gen_targets, gen_toy_stack
from tests.helpers import build_inputs, small_cfg
from tests.test_gpu_finetune import _row_check, _say, _tensor_check

pytestmark = pytest.mark.gpu

F64 = torch.float64


PRECISE = [
    # name, T, H_kv, H_q, B, N, n_s, step0, n_steps
    ("mha", 4, 2, 2, 2, 150, 4, 0, 4),
    ("gqa2-substeps", 4, 1, 2, 1, 97, 3, 1, 2),
    ("nosink", 4, 1, 1, 1, 70, 0, 0, 4),
]


@pytest.mark.parametrize("geo", PRECISE, ids=[p[0] for p in PRECISE])
def test_precise_attention_forward_backward(geo):
    name, T, H, Hq, B, N, n_s, step0, n_steps = geo
    _say("precise attention %s" % name)
    cfg = small_cfg(1, T=T, H_kv=H, H_q=Hq, B=B, N=N + 6, n_s=max(n_s, 1), rho_k=(0.85,) * (T - 1),
                    rho_v=(0.9,) * (T - 1))
    inp = build_inputs(cfg, 0, "cuda", kmeans=False)
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    rope = lv.rope_table_f32(n_s + cfg.N, cfg.D, cfg.theta)
    gq = torch.Generator(device="cpu").manual_seed(21)
    q = torch.randn((B, Hq, n_steps, N, cfg.D), generator=gq).cuda()
    dout = torch.randn((B, Hq, n_steps, N, cfg.D), generator=gq).cuda()
    sk = inp["sink_k"][:, :, :, :n_s].contiguous() if n_s else None
    sv = inp["sink_v"][:, :, :, :n_s].contiguous() if n_s else None
    k, v = inp["k"], inp["v"]                       # N_x = N + 6 tokens, N attended
    out, lse = lv.precise_attn(g, q, k, v, sk, sv, rope, step0=step0)
    d_k = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    d_v = torch.zeros_like(d_k)
    dq = lv.precise_attn_backward(g, q, k, v, sk, sv, rope, out, lse, dout, d_k, d_v, step0=step0)
    torch.cuda.synchronize()

    kr = k[:, :, :, :N].double().cpu().requires_grad_(True)
    vr = v[:, :, :, :N].double().cpu().requires_grad_(True)
    qr = q.double().cpu().requires_grad_(True)
    sks = (sk if n_s else inp["sink_k"][:, :, :, :0]).double().cpu()
    svs = (sv if n_s else inp["sink_v"][:, :, :, :0]).double().cpu()
    o_r = torch.empty((B, Hq, n_steps, N, cfg.D), dtype=F64)
    l_r = torch.empty((B, Hq, n_steps, N), dtype=F64)
    total = 0.0
    outs = []
    for b in range(B):
        for hq in range(Hq):
            h = hq // (Hq // H)
            for tl in range(n_steps):
                t = step0 + tl
                o, l = ref.causal_attention(qr[b, hq, tl], kr[b, h, t], vr[b, h, t], sks[b, h, t], svs[b, h, t],
                                            cfg.theta)
                outs.append((b, hq, tl, o, l))
                total = total + (o * dout[b, hq, tl].double().cpu()).sum()
    total.backward()
    for b, hq, tl, o, l in outs:
        o_r[b, hq, tl] = o.detach()
        l_r[b, hq, tl] = l.detach()
    _row_check(out, o_r, 1e-4, "out")
    assert float((lse.double().cpu() - l_r).abs().max()) <= 1e-4
    _row_check(dq, qr.grad, 1e-4, "d_q", floor=1e-2)
    gk = torch.zeros(k.shape, dtype=F64)
    gv = torch.zeros(k.shape, dtype=F64)
    gk[:, :, :, :N] = kr.grad
    gv[:, :, :, :N] = vr.grad
    _tensor_check(d_k, gk, 1e-4, "d_k")
    _tensor_check(d_v, gv, 1e-4, "d_v")
    # tokens past N and steps outside the range get nothing
    assert int(torch.count_nonzero(d_k[:, :, :, N:])) == 0
    served = torch.zeros(T, dtype=torch.bool)
    served[step0:step0 + n_steps] = True
    assert int(torch.count_nonzero(d_k[:, :, ~served.cuda()])) == 0


def _fisher_case(tasq, N=96, vocab=64):
    cfg = small_cfg(1, T=4, T_c=4, G=16, H_kv=2, H_q=2, B=2, N=N, n_s=4, tasq=tasq)
    inp = build_inputs(cfg, 0, "cuda", kmeans=False)
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    rope = lv.rope_table_f32(cfg.n_s + N, cfg.D, cfg.theta)
    toy = gen_toy_stack(cfg, 0, "cuda", vocab=vocab)
    y = gen_targets(cfg, 0, "cuda", vocab=vocab)
    stack = ft.ToyLoopedStack(toy["Wq"], toy["Wo"], toy["Wu"], cfg.H_q, cfg.D, cfg.T, cfg.n_s, rope)
    pt = sigma = None
    if tasq:
        # sigma of every token, written by the encode
        sigma = torch.zeros((cfg.B, N, cfg.T), dtype=torch.float16, device="cuda")
        pt = lv.pretransform(inp["w"], inp["perm"], sigma)
        idx = torch.zeros((cfg.B, cfg.H_kv, 1, N, cfg.chunks), dtype=torch.uint8, device="cuda")
        lv.encode(g, inp["k"], inp["k_cb"], idx, pt=pt)
    return cfg, g, inp, toy, y, stack, pt, sigma


@pytest.mark.parametrize("tasq", [False, True], ids=["plain", "pretransform"])
def test_fisher_weights_through_the_toy_stack(tasq):
    _say("importance weights, pre-transform=%s" % tasq)
    cfg, g, inp, toy, y, stack, pt, sigma = _fisher_case(tasq)
    L, ok, ov = ft.fisher_importance(stack, g, toy["x"], inp["k"], inp["v"], inp["sink_k"], inp["sink_v"], y, pt)
    torch.cuda.synchronize()
    t64 = {k: v.double().cpu() for k, v in toy.items()}
    cache = dict(k=inp["k"].double().cpu(), v=inp["v"].double().cpu(), sink_k=inp["sink_k"].double().cpu(),
                 sink_v=inp["sink_v"].double().cpu(), H_q=cfg.H_q, N=cfg.N)
    tq = None
    if tasq:
        tq = (inp["w"].double().cpu().numpy(), inp["perm"].long().cpu().numpy(), sigma.double().cpu().numpy())
    L_r, ok_r, ov_r = ref.fisher_importance(t64, cache, y.cpu().numpy(), cfg.T_c, cfg.G, cfg.theta, tq)
    _say("  loss %.9g (oracle %.9g)" % (L, L_r))
    assert abs(L - L_r) <= 1e-5 * abs(L_r)
    for name, got, want in (("omega_k", ok, ok_r), ("omega_v", ov, ov_r)):
        _tensor_check(got, torch.from_numpy(want), 2e-3, name)
        assert bool((got >= 0).all())


def test_fisher_weights_feed_the_weighted_kmeans():
    """One weighted k-means update with the GPU's weights equals the oracle's
    update with the oracle's weights on the same assignment, up to one bf16
    step where a quotient lands near a rounding midpoint."""
    cfg, g, inp, toy, y, stack, pt, sigma = _fisher_case(False)
    _, ok, _ = ft.fisher_importance(stack, g, toy["x"], inp["k"], inp["v"], inp["sink_k"], inp["sink_v"], y)
    idx = torch.zeros((cfg.B, cfg.H_kv, 1, cfg.N, cfg.chunks), dtype=torch.uint8, device="cuda")
    lv.encode(g, inp["k"], inp["k_cb"], idx)
    sums = torch.zeros((cfg.H_kv, 1, cfg.K, cfg.G), dtype=torch.float64, device="cuda")
    wsum = torch.zeros((cfg.H_kv, 1, cfg.K), dtype=torch.float64, device="cuda")
    lv.kmeans_accumulate(g, inp["k"], idx, sums, wsum, weight=ok.contiguous())
    cb = inp["k_cb"].clone()
    lv.kmeans_finalize(g, sums, wsum, cb)
    torch.cuda.synchronize()
    t64 = {k: v.double().cpu() for k, v in toy.items()}
    cache = dict(k=inp["k"].double().cpu(), v=inp["v"].double().cpu(), sink_k=inp["sink_k"].double().cpu(),
                 sink_v=inp["sink_v"].double().cpu(), H_q=cfg.H_q, N=cfg.N)
    _, ok_r, _ = ref.fisher_importance(t64, cache, y.cpu().numpy(), cfg.T_c, cfg.G, cfg.theta)
    kx = inp["k"].double().cpu().numpy()
    a_all = idx.long().cpu().numpy()
    for h in range(cfg.H_kv):
        z = np.concatenate([ref.joint_vectors(kx[b, h], cfg.T_c, cfg.G)[0].reshape(-1, cfg.G) for b in range(cfg.B)])
        om = np.concatenate([ok_r[b, h, 0].reshape(-1) for b in range(cfg.B)])
        asg = np.concatenate([a_all[b, h, 0].reshape(-1) for b in range(cfg.B)])
        _, sums_r, wsum_r = ref.weighted_kmeans_sums(z, om, inp["k_cb"][h, 0].double().cpu().numpy(), assign=asg)
        want = inp["k_cb"][h, 0].double().cpu().numpy().copy()
        nz = wsum_r > 0
        want[nz] = ref.bf16_round(sums_r[nz] / wsum_r[nz, None])
        got = cb[h, 0].double().cpu().numpy()
        diff = got != want
        # any difference is one bf16 step
        steps = np.abs(got[diff] - want[diff]) / np.maximum(np.abs(want[diff]), 1e-30)
        _say("  head %d: %d of %d entries differ" % (h, int(diff.sum()), diff.size))
        assert diff.mean() < 0.01 and np.all(steps <= 2 ** -7)
