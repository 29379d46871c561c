"""The allocation-free decode entry point (loopvq_decode_attn_noalloc, for
callers that cannot allocate device memory) against loopvq_decode_attn with a
caller workspace: identical outputs on two calls in a row, the second with a
smaller input, and a clear EWORKSPACE error for a shape whose split partials
exceed the static array."""
import sys

import pytest
import torch

from sub_bit_loop_amd import _lib as L
from tests.helpers import build_inputs, small_cfg

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _encoded(s, cfg):
    inp = build_inputs(cfg, 0, "cuda", kmeans=False)
    g = s.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    shp = (cfg.B, cfg.H_kv, cfg.n_blk, cfg.N, cfg.chunks)
    kidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    pt = None
    if cfg.tasq:
        sigma = torch.zeros((cfg.B, cfg.N, cfg.T), dtype=torch.float16, device="cuda")
        pt = s.pretransform(inp["w"], inp["perm"], sigma)
    s.encode(g, inp["k"], inp["k_cb"], kidx, pt=pt)
    s.encode(g, inp["v"], inp["v_cb"], vidx)
    rope = s.rope_table(cfg.n_s + cfg.N + 8, cfg.D, cfg.theta)
    return g, inp, kidx, vidx, pt, rope


CASES = [
    # name, then (geometry of the first call, geometry of the second, smaller call)
    ("pretransform", dict(G=16, T=4, H_kv=4, H_q=4, B=3, N=3000, tasq=True),
     dict(G=16, T=4, H_kv=2, H_q=2, B=2, N=700, tasq=True)),
    ("half-bit-mha", dict(G=16, T=4, H_kv=4, H_q=4, B=4, N=2500), dict(G=16, T=4, H_kv=4, H_q=4, B=1, N=300)),
    ("quarter-bit-gqa", dict(G=32, T=4, H_kv=2, H_q=8, B=2, N=2000), dict(G=32, T=4, H_kv=1, H_q=4, B=1, N=257)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_decode_equals_workspace_decode(case):
    import sub_bit_loop_amd as s
    s.lib()
    name, first, second = case
    for call, over in enumerate((first, second)):
        cfg = small_cfg(1, **over, rho_k=(0.85,) * (over["T"] - 1), rho_v=(0.9,) * (over["T"] - 1))
        _say("no-alloc decode", name, "call", call, over)
        g, inp, kidx, vidx, pt, rope = _encoded(s, cfg)
        for step0, n_steps, seq in ((0, cfg.T, None), (1, 1, None), (0, cfg.T, [cfg.N // 3] * cfg.B)):
            sl = None if seq is None else torch.tensor(seq, dtype=torch.int32, device="cuda")
            q = inp["q"][:, :, step0:step0 + n_steps].contiguous()
            o1, l1 = s.decode_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"], rope,
                                   step0=step0, seq_len=sl, pt=pt)
            out = torch.full_like(o1, float("nan"))
            lse = torch.full_like(l1, float("nan"))
            o2, l2 = s.decode_attn_noalloc(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"],
                                           inp["sink_v"], rope, step0=step0, seq_len=sl, pt=pt, out=out, lse=lse)
            torch.cuda.synchronize()
            assert o2.data_ptr() == out.data_ptr()
            assert torch.equal(o1, o2) and torch.equal(l1, l2), (name, call, step0, n_steps)


def test_noalloc_rejects_shapes_beyond_the_array():
    import sub_bit_loop_amd as s
    s.lib()
    # B * H_q * n_steps * n_split * (D + 1) * 4 bytes of partials above the limit
    cfg = small_cfg(1, G=16, T=4, H_kv=16, H_q=16, B=1100, N=16)
    g = s.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    assert s.decode_workspace_bytes(g, cfg.B, cfg.N, 0, cfg.T) > L.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((cfg.B, cfg.H_q, cfg.T, cfg.D), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((cfg.B, cfg.H_kv, cfg.n_blk, cfg.N, cfg.chunks), dtype=torch.uint8, device="cuda")
    cb = torch.zeros((cfg.H_kv, cfg.n_blk, cfg.K, cfg.G), dtype=torch.bfloat16, device="cuda")
    rope = s.rope_table(cfg.N + 8, cfg.D, cfg.theta)
    with pytest.raises(L.LoopVQError) as e:
        s.decode_attn_noalloc(g, q, idx, idx, cb, cb, None, None, rope)
    assert e.value.status == L.EWORKSPACE
