"""GPU: decode parity when the scores rise along the context.

Every decode kernel keeps an online-softmax running maximum that may lag the
true one by a few units and is raised (every partial sum rescaled) when a token
exceeds it.  Here the key codewords run along one direction from -amp to +amp,
the index of token n grows with n, and the queries live only in the RoPE pairs
of the four lowest frequencies (their angle stays below 0.2 rad over the
context), so the scores climb through zero by ~25 base-2 units over the context
and every lane raises its maximum about eight times, well past the first tokens.
The scores stay within about +-13 units: the fp16 score arithmetic carries an
absolute error that grows with the scores' magnitude, so logits of tens of nats
in a sharply peaked softmax would test that bound instead of the rescaling.  The
indices are built directly (no encode); both sides take the same ones, so the
check is the decode alone.
"""
import sys

import pytest
import torch

from tests.helpers import build_inputs, small_cfg
from tests.test_gpu_parity import _check_rows, _decode, _lib

pytestmark = pytest.mark.gpu

RISING = [
    # name, G, H_q, pretransform, n_steps (None: every step of the block)
    ("plain-c4", 16, 1, False, None),
    ("plain-c4-one-step", 16, 1, False, 1),
    ("plain-c8", 32, 1, False, None),
    ("gqa4-c4", 16, 4, False, None),
    ("pretransform-c4", 16, 1, True, None),
    ("pretransform-c4-one-step", 16, 1, True, 1),
    ("pretransform-c8", 32, 1, True, None),
]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("geo", RISING, ids=[x[0] for x in RISING])
def test_rising_scores(geo):
    s = _lib()
    name, G, Hq, tasq, n_steps = geo
    B, N, T, amp = 2, 1500, 4, 3.5
    _say("rising scores", name)
    cfg = small_cfg(1, G=G, T_c=4, T=T, H_kv=1, H_q=Hq, B=B, N=N, n_s=4, tasq=tasq,
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=2)
    inp = build_inputs(cfg, 0, "cuda")
    K, D = cfg.K, cfg.D
    # codeword r = amp * (2 r / (K - 1) - 1) in every joint coordinate
    ramp = (torch.arange(K, dtype=torch.float32, device="cuda") * (2.0 / (K - 1)) - 1.0) * amp
    inp["k_cb"] = ramp.view(1, 1, K, 1).expand(1, cfg.n_blk, K, G).to(torch.bfloat16).contiguous()
    # queries: amp on the pairs (60..63, 124..127) of every step, zero elsewhere
    q = torch.zeros((B, Hq, T, D), dtype=torch.float32, device="cuda")
    q[..., 60:64] = amp
    q[..., 124:128] = amp
    inp["q"] = q.to(torch.bfloat16)
    shp = (B, 1, cfg.n_blk, N, cfg.chunks)
    tok_idx = (torch.arange(N, device="cuda") * (K - 1) // (N - 1)).to(torch.uint8)
    kidx = tok_idx.view(1, 1, 1, N, 1).expand(shp).contiguous()
    gen = torch.Generator(device="cuda").manual_seed(7)
    vidx = torch.randint(0, K, shp, generator=gen, device="cuda").to(torch.uint8)
    sigma = pt = None
    if tasq:
        sigma = (0.5 + torch.rand((B, N, T), generator=gen, device="cuda")).to(torch.float16)
        pt = s.pretransform(inp["w"], inp["perm"], sigma)
    steps = [(0, T)] if n_steps is None else [(t, 1) for t in range(T)]
    worst = 0.0
    for t0, ns in steps:
        out, lse = _decode(s, cfg, inp, kidx, vidx, pt, step0=t0, n_steps=ns)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        rows = [(b, hq, t) for b in range(B) for hq in range(Hq) for t in range(t0, t0 + ns)]
        worst = max(worst, _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows, step0=t0))
    _say("  worst rel err %.3g, lse %.1f .. %.1f" % (worst, lse.min().item(), lse.max().item()))
