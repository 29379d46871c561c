"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times, checked against the fp64 oracle on sampled slices:
seeded (batch, kv-head) encode slices over first, last and random tokens, and
seeded decode rows over the whole context (sinks included), for the fused call
over all steps and, on workloads 2 and 3, for a per-step call."""
import numpy as np
import pytest
import torch

import oracle as ref
from synth import config_by_index
from tests.helpers import OUT_TOL, build_inputs, check_indices, np64, row_error
from tests.test_gpu_parity import _check_encode_slice, _check_rows, _decode, _encode_all, _geom, _lib, _say

pytestmark = pytest.mark.gpu


def _token_sample(N, rng, n=256):
    toks = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N), rng.integers(0, N, n - 128)]))
    return toks


def _run_config(idx, n_enc=3, n_rows=8, layer=0):
    s = _lib()
    cfg = config_by_index(idx)
    rng = np.random.default_rng(1000 + idx)
    _say("config %d layer %d: generating inputs" % (idx, layer))
    inp = build_inputs(cfg, layer, "cuda")
    kidx, vidx, sigma, pt = _encode_all(s, cfg, inp, N_cap=cfg.N + cfg.page * (cfg.decode_steps // cfg.page))
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, N=cfg.N)
    torch.cuda.synchronize()
    _say("config %d: GPU done, checking" % idx)
    fails = 0
    for _ in range(n_enc):
        b, h = int(rng.integers(cfg.B)), int(rng.integers(cfg.H_kv))
        toks = _token_sample(cfg.N, rng)
        rk, rv = _check_encode_slice(cfg, inp, kidx[:, :, :, :cfg.N], vidx[:, :, :, :cfg.N], sigma, b, h, toks)
        _say("  encode b%d h%d K exact/tie/fail %s V %s" % (b, h, rk, rv))
        fails += rk[2] + rv[2]
    assert fails == 0
    rows = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.H_q)), int(rng.integers(cfg.T))) for _ in range(n_rows)]
    rows += [(0, 0, 0), (cfg.B - 1, cfg.H_q - 1, cfg.T - 1)]
    worst = _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows, N=cfg.N)
    _say("  decode worst rel err %.3g over %d rows (tolerance %g)" % (worst, len(rows), OUT_TOL))
    return s, cfg, inp, kidx, vidx, sigma, pt


def _per_step_call(s, cfg, inp, kidx, vidx, sigma, pt, t, seed, n_rows=6):
    """One decode call for loop step t alone (n_steps = 1), the per-step use."""
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, N=cfg.N, step0=t, n_steps=1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.H_q)), t) for _ in range(n_rows)]
    worst = _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows, step0=t, N=cfg.N)
    _say("  per-step call (step %d): decode worst rel err %.3g" % (t, worst))


def test_config1_full():
    _run_config(1, n_rows=4)


def test_config2_full():
    s, cfg, inp, kidx, vidx, sigma, pt = _run_config(2)
    _per_step_call(s, cfg, inp, kidx, vidx, sigma, pt, 1, 2002)


def test_config3_full():
    s, cfg, inp, kidx, vidx, sigma, pt = _run_config(3)
    _per_step_call(s, cfg, inp, kidx, vidx, sigma, pt, 2, 3003)


def test_config4_full():
    _run_config(4, n_rows=12)


@pytest.mark.parametrize("layer", [0, 23])
def test_config5_layer_with_page_encode(layer):
    s, cfg, inp, kidx, vidx, sigma, pt = _run_config(5, n_enc=2, n_rows=6, layer=layer)
    # one decode-time page event: 8 more tokens appended at token N
    from synth.generator import gen_kv_layer
    g = _geom(s, cfg)
    page_k = inp["k"][:, :, :, -cfg.page:].clone()
    page_v = inp["v"][:, :, :, -cfg.page:].clone()
    s.encode(g, page_k, inp["k_cb"], kidx, tok0=cfg.N, pt=pt)
    s.encode(g, page_v, inp["v_cb"], vidx, tok0=cfg.N)
    torch.cuda.synchronize()
    # the appended rows must equal the rows of the same tokens at their original place
    assert torch.equal(kidx[:, :, :, cfg.N:cfg.N + cfg.page], kidx[:, :, :, cfg.N - cfg.page:cfg.N])
    assert torch.equal(vidx[:, :, :, cfg.N:cfg.N + cfg.page], vidx[:, :, :, cfg.N - cfg.page:cfg.N])
    assert torch.equal(sigma[:, cfg.N:cfg.N + cfg.page], sigma[:, cfg.N - cfg.page:cfg.N])
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, N=cfg.N + cfg.page)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77 + layer)
    rows = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.H_q)), int(rng.integers(cfg.T))) for _ in range(4)]
    worst = _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows, N=cfg.N + cfg.page)
    _say("  after page encode: decode worst rel err %.3g" % worst)
