"""GPU: loopvq_decode_attn with lse = NULL (the C ABI allows it) writes the
same out as the call that also returns lse, on the kernel paths that write
out themselves (one context split: the pre-transform, c = 4 multi-step and
GQA kernels) and on the path through the merge kernel (several splits)."""
import ctypes

import pytest
import torch

from tests.helpers import build_inputs, small_cfg
from tests.test_gpu_parity import _encode_all, _geom, _lib, _say

pytestmark = pytest.mark.gpu

CASES = [
    # name, G, H_kv, H_q, N, pretransform
    ("pretransform-one-split", 16, 2, 2, 200, True),
    ("c4-mha-one-split", 16, 1, 1, 200, False),
    ("gqa4-one-split", 32, 1, 4, 200, False),
    ("pretransform-splits", 16, 2, 2, 700, True),
    ("c4-mha-splits", 16, 1, 1, 700, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_without_lse(case):
    s = _lib()
    name, G, H, Hq, N, tasq = case
    _say("null lse", name)
    cfg = small_cfg(1, G=G, T_c=4, T=4, H_kv=H, H_q=Hq, B=2, N=N, n_s=4, tasq=tasq,
                    rho_k=(0.85,) * 3, rho_v=(0.9,) * 3, n_calib=1024, kmeans_iters=3)
    inp = build_inputs(cfg, 0, "cuda")
    kidx, vidx, sigma, pt = _encode_all(s, cfg, inp)
    g = _geom(s, cfg)
    rope = s.rope_table(cfg.n_s + N + 8, cfg.D, cfg.theta)
    out1, lse1 = s.decode_attn(g, inp["q"], kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"],
                               rope, N=N, pt=pt)
    need = s.decode_workspace_bytes(g, cfg.B, N, 0, cfg.T)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    out2 = torch.full_like(out1, float("nan"))
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    from sub_bit_loop_amd import _lib as L
    st = L.lib().loopvq_decode_attn(
        ctypes.byref(g), P(inp["q"]), 0, cfg.T, P(kidx), P(vidx), N, P(inp["k_cb"]), P(inp["v_cb"]),
        P(inp["sink_k"]), P(inp["sink_v"]), cfg.n_s, None, None, 0, 0, cfg.B, N, None,
        ctypes.byref(pt) if pt is not None else None, P(rope), rope.shape[0], P(out2), None, P(ws),
        ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.lib().loopvq_last_error()
    torch.cuda.synchronize()
    assert torch.isfinite(lse1).all()
    assert torch.equal(out1, out2)
