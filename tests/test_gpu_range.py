"""GPU: input range of the fp16 decode kernels.

The fast decode kernels work in fp16 after power-of-two rescaling of the
queries, of the key codebooks together with the bf16 sinks and recent keys,
and of the values.  Two checks per kernel:

* invariance: q * 2^20 with every key (codebooks, sinks, recent window) *
  2^-20 leaves the scores unchanged, and values * 2^20 scale the output by
  2^20.  Power-of-two scales commute with every fp16/fp32 rounding the kernels
  do, so the result must be bit-identical to the unscaled run times 2^20 (the
  log-sum-exp bit-identical), and it must also match the oracle.  Without the
  query scale |q| ~ 1e6 overflows fp16.
* sink-dominated range: sinks and recent keys * 2^16 with queries * 2^-16
  (and sink/recent values * 2^10) against the oracle: the bf16 rows must
  count in the codebooks' range (else they overflow fp16) and small queries
  must be scaled up (else they fall into fp16 subnormals).
"""
import sys

import pytest
import torch

from tests.helpers import build_inputs, small_cfg
from tests.test_gpu_parity import _check_rows, _decode, _encode_all, _lib

pytestmark = pytest.mark.gpu

RANGE_GEOMS = [
    # name, G, T, T_c, H_kv, H_q, pretransform, n_steps (None: every step)
    ("multi-step-c4", 16, 8, 4, 1, 1, False, None),
    ("multi-step-c8", 32, 4, 4, 1, 1, False, None),
    ("single-step-c4", 16, 4, 4, 1, 1, False, 1),
    ("gqa2-c4", 16, 4, 4, 1, 2, False, None),
    ("gqa4-c8", 32, 4, 4, 1, 4, False, None),
    ("gqa4-one-step", 16, 4, 4, 1, 4, False, 1),
    ("pretransform-c4", 16, 4, 4, 1, 1, True, None),
    ("pretransform-c8", 32, 4, 4, 1, 1, True, None),
    ("pretransform-one-step-c4", 16, 4, 4, 1, 1, True, 1),
    ("pretransform-one-step-c8", 32, 4, 4, 1, 1, True, 1),
    ("per-step-codebooks", 16, 4, 1, 1, 1, False, None),
    ("generic-tc2", 16, 4, 2, 1, 1, False, None),
]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _scaled(x, e):
    return None if x is None else (x.float() * 2.0 ** e).to(torch.bfloat16)


@pytest.mark.parametrize("geo", RANGE_GEOMS, ids=[x[0] for x in RANGE_GEOMS])
def test_input_range_scaling(geo):
    s = _lib()
    name, G, T, T_c, H, Hq, tasq, n_steps = geo
    B, N, n_r = 2, 300, 5
    _say("input range", name)
    cfg = small_cfg(1, G=G, T_c=T_c, T=T, H_kv=H, H_q=Hq, B=B, N=N + n_r, n_s=4, tasq=tasq,
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=5)
    inp = build_inputs(cfg, 0, "cuda")
    recent = (inp["k"][:, :, :, N:].contiguous(), inp["v"][:, :, :, N:].contiguous())
    inp = dict(inp, k=inp["k"][:, :, :, :N].contiguous(), v=inp["v"][:, :, :, :N].contiguous())
    kidx, vidx, sigma, pt = _encode_all(s, cfg, inp)
    steps = [(0, T)] if n_steps is None else [(t, 1) for t in range(T)]

    def run(x, rec):
        res = [_decode(s, cfg, x, kidx, vidx, pt, step0=t0, n_steps=ns, recent=rec) for t0, ns in steps]
        torch.cuda.synchronize()
        return res

    def check(x, rec, res):
        worst = 0.0
        for (t0, ns), (out, lse) in zip(steps, res):
            assert torch.isfinite(out).all() and torch.isfinite(lse).all()
            rows = [(b, hq, t) for b in range(B) for hq in range(Hq) for t in range(t0, t0 + ns)]
            worst = max(worst, _check_rows(cfg, x, kidx, vidx, sigma, out, lse, rows, step0=t0, recent=rec))
        return worst

    base = run(inp, recent)
    w0 = check(inp, recent, base)

    # invariance under q * 2^20, keys * 2^-20, values * 2^20
    E = 20
    inp_a = dict(inp, q=_scaled(inp["q"], E), k_cb=_scaled(inp["k_cb"], -E), sink_k=_scaled(inp["sink_k"], -E),
                 v_cb=_scaled(inp["v_cb"], E), sink_v=_scaled(inp["sink_v"], E))
    rec_a = (_scaled(recent[0], -E), _scaled(recent[1], E))
    assert inp_a["q"].float().abs().max().item() > 65504.0    # beyond fp16 without a scale
    res_a = run(inp_a, rec_a)
    for (o0, l0), (o1, l1) in zip(base, res_a):
        assert torch.equal(o1, o0 * 2.0 ** E), (o1 / 2.0 ** E - o0).abs().max().item()
        assert torch.equal(l1, l0)
    w1 = check(inp_a, rec_a, res_a)

    # sink-dominated ranges, small queries
    inp_b = dict(inp, q=_scaled(inp["q"], -16), sink_k=_scaled(inp["sink_k"], 16),
                 sink_v=_scaled(inp["sink_v"], 10))
    rec_b = (_scaled(recent[0], 16), _scaled(recent[1], 10))
    assert inp_b["sink_k"].float().abs().max().item() > 65504.0
    res_b = run(inp_b, rec_b)
    w2 = check(inp_b, rec_b, res_b)
    _say("  worst rel err %.3g plain, %.3g scaled, %.3g sink-dominated" % (w0, w1, w2))
