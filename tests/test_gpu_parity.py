"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Indices must equal the oracle's wherever the oracle's tie set has one element
and lie in the tie set elsewhere; decode outputs must satisfy
max_d |o_gpu - o_ref| <= 2e-3 * ||o_ref||_2 per (batch, q-head, step) row.
Decode parity feeds both sides the GPU's own index tensors.
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import oracle as ref
from synth import config_by_index
from tests.helpers import (OUT_TOL, build_inputs, check_indices, np64, row_error, small_cfg)

pytestmark = pytest.mark.gpu


def _lib():
    import sub_bit_loop_amd as s
    s.lib()
    return s


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _geom(s, cfg):
    return s.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)


def _encode_all(s, cfg, inp, N_cap=None, pt_sigma=None):
    g = _geom(s, cfg)
    N = inp["k"].shape[3]
    B = inp["k"].shape[0]
    N_cap = N if N_cap is None else N_cap
    shp = (B, cfg.H_kv, cfg.n_blk, N_cap, cfg.chunks)
    kidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    pt = None
    sigma = None
    if cfg.tasq:
        sigma = torch.zeros((B, N_cap, cfg.T), dtype=torch.float16, device="cuda")
        pt = s.pretransform(inp["w"], inp["perm"], sigma)
    s.encode(g, inp["k"], inp["k_cb"], kidx, pt=pt)
    s.encode(g, inp["v"], inp["v_cb"], vidx)
    return kidx, vidx, sigma, pt


def _check_encode_slice(cfg, inp, kidx, vidx, sigma, b, h, toks):
    """Oracle check of one (batch, kv-head) over a token subset."""
    kx = np64(inp["k"][b, h][:, toks])
    vx = np64(inp["v"][b, h][:, toks])
    kc = np64(inp["k_cb"][h])
    vc = np64(inp["v_cb"][h])
    gk = kidx[b, h][:, toks].cpu().numpy()
    gv = vidx[b, h][:, toks].cpu().numpy()
    tasq = None
    if cfg.tasq:
        klayer = np64(inp["k"][b][:, :, toks])           # [H, T, n, D]
        sig_ref = ref.tasq_sigma(klayer)                  # [n, T]
        sbar = ref.fp16_round(sig_ref)
        sg = sigma[b, toks].double().cpu().numpy()
        # fp16 rounding must agree except within 1e-6 relative of a midpoint
        mism = sg != sbar
        if mism.any():
            lo = ref.fp16_round(sig_ref * (1 - 1e-6))
            hi = ref.fp16_round(sig_ref * (1 + 1e-6))
            assert np.all((lo != hi)[mism]), "sigma differs from the oracle's fp16 rounding"
        w = inp["w"][h].double().cpu().numpy()
        perm = inp["perm"][h].long().cpu().numpy()
        tasq = (w, perm, sg)
    rk = check_indices(gk, kx, kc, cfg.T_c, tasq)
    rv = check_indices(gv, vx, vc, cfg.T_c)
    return rk, rv


def _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows, step0=0, N=None, seq=None, recent=None, errs=None):
    """rows: list of (b, hq, t) with t absolute step; out/lse hold steps from step0.
    Returns the worst row error; appends every row's error to errs when given."""
    worst = 0.0
    gqa = cfg.H_q // cfg.H_kv
    for (b, hq, t) in rows:
        h = hq // gqa
        Nb = kidx.shape[3] if N is None else N
        if seq is not None:
            Nb = max(0, min(int(seq[b]), Nb))
        ki = kidx[b, h].cpu().numpy()
        vi = vidx[b, h].cpu().numpy()
        tasq = None
        if cfg.tasq:
            tasq = (inp["w"][h].double().cpu().numpy(), inp["perm"][h].long().cpu().numpy(),
                    sigma[b].double().cpu().numpy())
        q = np64(inp["q"][b, hq, t])            # inp["q"] holds every step
        n_s = inp["sink_k"].shape[3] if inp["sink_k"] is not None else 0
        sk = np64(inp["sink_k"][b, h]) if n_s else np.zeros((cfg.T, 0, cfg.D))
        sv = np64(inp["sink_v"][b, h]) if n_s else np.zeros((cfg.T, 0, cfg.D))
        o_gpu = out[b, hq, t - step0].double().cpu().numpy()
        n_r = 0 if recent is None else recent[0].shape[3]
        if Nb + n_s + n_r == 0:
            assert np.all(o_gpu == 0) and lse[b, hq, t - step0].item() == -math.inf
            continue
        rk = rv = None
        if recent is not None:
            rk, rv = np64(recent[0][b, h]), np64(recent[1][b, h])
        o_ref, l_ref = ref.decode_attn_row(q, t, ki, vi, np64(inp["k_cb"][h]), np64(inp["v_cb"][h]),
                                           sk, sv, cfg.T_c, cfg.theta, n_tokens=Nb, tasq=tasq,
                                           recent_k=rk, recent_v=rv)
        err = row_error(o_gpu, o_ref)
        worst = max(worst, err)
        if errs is not None:
            errs.append(err)
        assert err <= OUT_TOL, "row %s: err %.3g" % ((b, hq, t), err)
        assert abs(lse[b, hq, t - step0].item() - l_ref) < 1e-3 * max(1.0, abs(l_ref))
    return worst


def _decode(s, cfg, inp, kidx, vidx, pt, N=None, step0=0, n_steps=None, seq=None, n_s=None, recent=None):
    g = _geom(s, cfg)
    n_steps = cfg.T if n_steps is None else n_steps
    N = kidx.shape[3] if N is None else N
    ns = inp["sink_k"].shape[3] if n_s is None else n_s
    n_r = 0 if recent is None else recent[0].shape[3]
    rope = s.rope_table(ns + kidx.shape[3] + n_r + 8, cfg.D, cfg.theta)
    q = inp["q"][:, :, step0:step0 + n_steps].contiguous()
    sk = inp["sink_k"] if ns else None
    sv = inp["sink_v"] if ns else None
    rk, rv = (None, None) if recent is None else recent
    return s.decode_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, N=N, step0=step0,
                         seq_len=seq, pt=pt, recent_k=rk, recent_v=rv)


def test_config1_full():
    s = _lib()
    cfg = config_by_index(1)
    _say("config 1: building inputs")
    inp = build_inputs(cfg, 0, "cuda")
    kidx, vidx, sigma, pt = _encode_all(s, cfg, inp)
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt)
    torch.cuda.synchronize()
    rk, rv = _check_encode_slice(cfg, inp, kidx, vidx, sigma, 0, 0, slice(None))
    _say("config 1 encode K exact/tie/fail", rk, "V", rv)
    assert rk[2] == 0 and rv[2] == 0
    rows = [(0, 0, t) for t in range(cfg.T)]
    worst = _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows)
    _say("config 1 decode worst rel err %.3g" % worst)


GEOMS = [
    # name, G, T_c, T, H_kv, H_q, B, N, n_s, K, tasq
    ("two-blocks-gqa2", 16, 4, 8, 2, 4, 2, 1000, 4, 256, False),
    ("quarter-bit-gqa4", 32, 4, 4, 2, 8, 2, 701, 4, 256, False),
    ("half-bit-gqa4", 16, 4, 4, 1, 4, 2, 555, 4, 256, False),
    ("quarter-bit-gqa8", 32, 4, 4, 1, 8, 1, 333, 4, 256, False),
    ("quarter-bit-mha", 32, 4, 4, 2, 2, 2, 650, 4, 256, False),
    ("quarter-bit-2blk-gqa2", 32, 4, 8, 1, 2, 1, 480, 4, 256, False),
    ("pretransform", 16, 4, 4, 2, 2, 2, 777, 4, 256, True),
    ("pretransform-quarter-bit", 32, 4, 4, 2, 2, 1, 600, 4, 256, True),
    ("pretransform-2blk-gqa2", 16, 4, 8, 1, 2, 2, 500, 4, 256, True),
    ("pretransform-k200-nosink", 16, 4, 4, 1, 1, 2, 333, 0, 200, True),
    # one context split: the pre-transform kernel writes out / lse itself
    ("pretransform-one-split", 16, 4, 4, 2, 2, 2, 200, 4, 256, True),
    ("tc2-k200-nosink", 16, 2, 4, 1, 1, 1, 300, 0, 200, False),
    ("tc1-channel-vq", 16, 1, 2, 1, 2, 1, 129, 3, 64, False),
    ("tc8", 32, 8, 8, 1, 1, 1, 200, 2, 256, False),
]


@pytest.mark.parametrize("geo", GEOMS, ids=[x[0] for x in GEOMS])
def test_small_geometries(geo):
    s = _lib()
    name, G, T_c, T, H, Hq, B, N, n_s, K, tasq = geo
    _say("geometry", name)
    cfg = small_cfg(1, G=G, T_c=T_c, T=T, H_kv=H, H_q=Hq, B=B, N=N, n_s=n_s, K=K, tasq=tasq,
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=8)
    inp = build_inputs(cfg, 0, "cuda", kmeans=True)
    # plant exact codewords and duplicate codewords to exercise exact ties: row
    # K-1 copies row 3 (another group of four candidates), row 6 copies row 4
    # (the same group)
    kc = inp["k_cb"]
    kc[:, :, K - 1] = kc[:, :, 3]
    if K >= 8:
        kc[:, :, 6] = kc[:, :, 4]
    c = cfg.c
    planted = [] if tasq else [(j, (j * 37) % K) for j in range(0, min(N, 40), 7)]
    if not tasq and K >= 8:
        planted += [(1, 6), (2, 4)]
    for j, r in planted:
        for beta in range(cfg.n_blk):
            for m in range(T_c):
                for i in range(c):
                    val = kc[:, beta, r, i * T_c + m].view(1, H, 1).expand(B, H, cfg.D // c)
                    inp["k"][:, :, beta * T_c + m, j, i::c] = val
    kidx, vidx, sigma, pt = _encode_all(s, cfg, inp)
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, n_s=n_s)
    torch.cuda.synchronize()
    fails = 0
    for b in range(B):
        for h in range(H):
            rk, rv = _check_encode_slice(cfg, inp, kidx, vidx, sigma, b, h, slice(None))
            fails += rk[2] + rv[2]
            _say("  b%d h%d K exact/tie/fail %s V %s" % (b, h, rk, rv))
    assert fails == 0
    # a token planted on codeword r encodes every chunk to the lowest index
    # whose codeword equals row r (the argmin's tie rule)
    kcc = kc.cpu()
    kic = kidx.cpu()
    for j, r in planted:
        for h in range(H):
            for beta in range(cfg.n_blk):
                same = [rr for rr in range(K) if torch.equal(kcc[h, beta, rr], kcc[h, beta, r])]
                assert bool((kic[:, h, beta, j] == same[0]).all()), (j, r, h, beta, same[0])
    rows = [(b, hq, t) for b in range(B) for hq in range(Hq) for t in range(T)]
    worst = _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows)
    _say("  decode worst rel err %.3g over %d rows" % (worst, len(rows)))


EDGE_GEOMS = [
    # name, G, T, T_c, H_kv, H_q, pretransform  (the plain multi-step kernel, the GQA
    # MFMA kernel with four and two q-heads per workgroup, the pre-transform kernel and
    # the per-step-codebook kernel; T = 8 gives ranges that cross a block boundary)
    ("mha", 16, 4, 4, 1, 1, False),
    ("gqa4-2blk", 32, 8, 4, 1, 4, False),
    ("gqa2-2blk", 16, 8, 4, 1, 2, False),
    ("pretransform-2blk", 16, 8, 4, 1, 1, True),
    ("per-step-codebooks", 16, 8, 1, 1, 2, False),
]


@pytest.mark.parametrize("geo", EDGE_GEOMS, ids=[x[0] for x in EDGE_GEOMS])
def test_edge_cases(geo):
    s = _lib()
    name, G, T, T_c, H, Hq, tasq = geo
    _say("edge cases", name)
    cfg = small_cfg(1, G=G, T=T, T_c=T_c, B=3, N=300, H_kv=H, H_q=Hq, tasq=tasq, rho_k=(0.85,) * (T - 1),
                    rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=5)
    inp = build_inputs(cfg, 0, "cuda")
    kidx, vidx, sigma, pt = _encode_all(s, cfg, inp)
    all_rows = [(b, hq, t) for b in range(3) for hq in range(Hq) for t in range(T)]
    # only sinks (N = 0)
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, N=0)
    torch.cuda.synchronize()
    _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, all_rows, N=0)
    # per-batch lengths, one row with no keys at all
    seq = torch.tensor([0, 5, 1000], dtype=torch.int32, device="cuda")
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, seq=seq, n_s=0)
    torch.cuda.synchronize()
    inp0 = dict(inp, sink_k=None, sink_v=None)
    _check_rows(cfg, inp0, kidx, vidx, sigma, out, lse, all_rows, seq=seq.cpu().numpy())
    # step sub-ranges: one step, a middle pair, and (T = 8) ranges across the block boundary
    ranges = [(2, 1), (1, 2)] + ([(3, 2), (2, 5), (5, 3)] if T == 8 else [])
    for step0, n_steps in ranges:
        out, lse = _decode(s, cfg, inp, kidx, vidx, pt, step0=step0, n_steps=n_steps)
        torch.cuda.synchronize()
        _check_rows(cfg, inp, kidx, vidx, sigma, out, lse,
                    [(b, hq, t) for b in range(3) for hq in range(Hq) for t in range(step0, step0 + n_steps)],
                    step0=step0)
    # append: encode tokens [200, 300) at tok0 = 200 into a fresh buffer
    g = _geom(s, cfg)
    idx2 = torch.zeros_like(kidx)
    idx2[:, :, :, :200] = kidx[:, :, :, :200]
    s.encode(g, inp["k"][:, :, :, 200:], inp["k_cb"], idx2, tok0=200, pt=pt)
    torch.cuda.synchronize()
    assert torch.equal(idx2, kidx)
    # determinism: identical bytes on a second run
    k2, v2, _, _ = _encode_all(s, cfg, inp)
    o2, l2 = _decode(s, cfg, inp, k2, v2, pt)
    o1, l1 = _decode(s, cfg, inp, kidx, vidx, pt)
    torch.cuda.synchronize()
    assert torch.equal(k2, kidx) and torch.equal(v2, vidx)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_rope_table_matches_oracle():
    s = _lib()
    t = s.rope_table(65800, 128, 1.0e4)
    torch.cuda.synchronize()
    tab = ref.rope_table(65800, 128)                       # [pos][64][cos, sin] fp64
    got = t.double().cpu().numpy().reshape(65800, 16, 2, 4)
    cos = got[:, :, 0, :].reshape(65800, 64)
    sin = got[:, :, 1, :].reshape(65800, 64)
    # one fp16 rounding of a value in [-1, 1]: at most half an ulp of 2^-11
    assert np.max(np.abs(cos - tab[:, :, 0])) <= 2.0 ** -12
    assert np.max(np.abs(sin - tab[:, :, 1])) <= 2.0 ** -12
    want = ref.fp16_round(tab[:, :, 0])
    assert np.mean(cos == want) > 0.999


RECENT = [
    # name, G, T_c, T, H_kv, H_q, B, N, n_r, pretransform
    ("half-bit", 16, 4, 4, 2, 2, 2, 600, 64, False),
    ("quarter-bit-gqa", 32, 4, 4, 1, 4, 2, 500, 64, False),
    ("generic-tc2", 16, 2, 4, 1, 1, 2, 300, 24, False),
    ("per-step-codebooks", 16, 1, 4, 2, 2, 2, 300, 24, False),
    ("pretransform", 16, 4, 4, 2, 2, 1, 400, 32, True),
]


@pytest.mark.parametrize("geo", RECENT, ids=[x[0] for x in RECENT])
def test_recent_window_and_page_conversion(geo):
    """bf16 recent window in the same softmax, then one 8-token page moved from
    the window into the compressed cache (encode at tok0 = N)."""
    s = _lib()
    name, G, T_c, T, H, Hq, B, N, n_r, tasq = geo
    _say("recent window", name)
    cfg = small_cfg(1, G=G, T_c=T_c, T=T, H_kv=H, H_q=Hq, B=B, N=N + n_r, n_s=4, tasq=tasq,
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=8)
    inp = build_inputs(cfg, 0, "cuda")
    g = _geom(s, cfg)
    cap = N + n_r
    shp = (B, H, cfg.n_blk, cap, cfg.chunks)
    kidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    sigma = None
    pt = None
    if tasq:
        sigma = torch.zeros((B, cap, T), dtype=torch.float16, device="cuda")
        pt = s.pretransform(inp["w"], inp["perm"], sigma)
    s.encode(g, inp["k"][:, :, :, :N], inp["k_cb"], kidx, pt=pt)
    s.encode(g, inp["v"][:, :, :, :N], inp["v_cb"], vidx)
    rk = inp["k"][:, :, :, N:].contiguous()
    rv = inp["v"][:, :, :, N:].contiguous()
    rows = [(b, hq, t) for b in range(B) for hq in range(Hq) for t in range(T)]
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, N=N, recent=(rk, rv))
    torch.cuda.synchronize()
    w1 = _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows, N=N, recent=(rk, rv))
    # page conversion: the oldest 8 recent tokens become codes at tok0 = N
    s.encode(g, rk[:, :, :, :8], inp["k_cb"], kidx, tok0=N, pt=pt)
    s.encode(g, rv[:, :, :, :8], inp["v_cb"], vidx, tok0=N)
    rk2, rv2 = rk[:, :, :, 8:].contiguous(), rv[:, :, :, 8:].contiguous()
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt, N=N + 8, recent=(rk2, rv2))
    torch.cuda.synchronize()
    w2 = _check_rows(cfg, inp, kidx, vidx, sigma, out, lse, rows, N=N + 8, recent=(rk2, rv2))
    _say("  worst rel err %.3g before, %.3g after the page conversion" % (w1, w2))


STEP_GEOMS = [
    # name, G, T, H_kv, H_q, B, N, n_s, n_r, pretransform
    ("half-bit-2blk-gqa2", 16, 8, 2, 4, 2, 700, 4, 0, False),
    ("quarter-bit-gqa4-recent", 32, 4, 2, 8, 2, 513, 4, 40, False),
    ("half-bit-nosink-recent", 16, 4, 1, 1, 3, 300, 0, 24, False),
    ("pretransform-recent", 16, 4, 2, 2, 2, 450, 4, 16, True),
]


@pytest.mark.parametrize("geo", STEP_GEOMS, ids=[x[0] for x in STEP_GEOMS])
def test_per_step_decode(geo):
    """One call per loop step (n_steps = 1), as a looped model runs its steps
    in sequence: every row against the oracle, with per-batch lengths (one
    batch entry with no quantized tokens), and against the fused call."""
    s = _lib()
    name, G, T, H, Hq, B, N, n_s, n_r, tasq = geo
    _say("per-step decode", name)
    cfg = small_cfg(1, G=G, T_c=4, T=T, H_kv=H, H_q=Hq, B=B, N=N + n_r, n_s=n_s, tasq=tasq,
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=8)
    inp = build_inputs(cfg, 0, "cuda")
    g = _geom(s, cfg)
    shp = (B, H, cfg.n_blk, N, cfg.chunks)
    kidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    pt = sigma = None
    if tasq:
        sigma = torch.zeros((B, N, T), dtype=torch.float16, device="cuda")
        pt = s.pretransform(inp["w"], inp["perm"], sigma)
    s.encode(g, inp["k"][:, :, :, :N], inp["k_cb"], kidx, pt=pt)
    s.encode(g, inp["v"][:, :, :, :N], inp["v_cb"], vidx)
    recent = None
    if n_r:
        recent = (inp["k"][:, :, :, N:].contiguous(), inp["v"][:, :, :, N:].contiguous())
    seq = torch.tensor([N, 0, N - 77][:B], dtype=torch.int32, device="cuda")
    fused, fused_lse = _decode(s, cfg, inp, kidx, vidx, pt, N=N, seq=seq, n_s=n_s, recent=recent)
    worst = 0.0
    for t in range(T):
        out, lse = _decode(s, cfg, inp, kidx, vidx, pt, N=N, step0=t, n_steps=1, seq=seq, n_s=n_s,
                           recent=recent)
        torch.cuda.synchronize()
        rows = [(b, hq, t) for b in range(B) for hq in range(Hq)]
        inp_rows = inp if n_s else dict(inp, sink_k=None, sink_v=None)
        worst = max(worst, _check_rows(cfg, inp_rows, kidx, vidx, sigma, out, lse, rows, step0=t,
                                       seq=seq.cpu().numpy(), recent=recent))
        # the single-step and the fused kernels agree within their fp16 rounding
        d = (out[:, :, 0] - fused[:, :, t]).abs().max().item()
        scale = fused[:, :, t].abs().max().item()
        assert d <= 4 * OUT_TOL * max(scale, 1e-30), (t, d, scale)
        fin = torch.isfinite(fused_lse[:, :, t])
        assert torch.equal(fin, torch.isfinite(lse[:, :, 0]))
        assert torch.allclose(lse[:, :, 0][fin], fused_lse[:, :, t][fin], atol=1e-3, rtol=1e-4)
    _say("  decode worst rel err %.3g over %d steps" % (worst, T))


SHORT = [
    # name, G, pretransform: c = 4 (32 codes per token) and c = 8 (16 per token)
    ("half-bit", 16, False),
    ("quarter-bit", 32, False),
    ("pretransform", 16, True),
    ("pretransform-quarter-bit", 32, True),
]


@pytest.mark.parametrize("geo", SHORT, ids=[x[0] for x in SHORT])
def test_encode_exactly_sized_short_inputs(geo):
    """Encodes of 1, 2, 3, 129 and 130 tokens from tensors holding exactly those
    tokens (and a sigma buffer of exactly N tokens): the last workgroup has fewer
    groups of codes than waves, and every load must stay inside the inputs."""
    s = _lib()
    name, G, tasq = geo
    for N in (1, 2, 3, 129, 130):
        _say("short encode", name, "N=%d" % N)
        cfg = small_cfg(1, G=G, T_c=4, T=4, H_kv=2, H_q=2, B=2, N=N, n_s=4, tasq=tasq,
                        n_calib=1024, kmeans_iters=4)
        inp = build_inputs(cfg, 0, "cuda")
        x = inp["k"].contiguous()
        assert x.shape[3] == N
        g = _geom(s, cfg)
        kidx = torch.zeros((2, 2, 1, N, cfg.chunks), dtype=torch.uint8, device="cuda")
        pt = sigma = None
        if tasq:
            sigma = torch.zeros((2, N, 4), dtype=torch.float16, device="cuda")
            pt = s.pretransform(inp["w"], inp["perm"], sigma)
        vidx = torch.zeros_like(kidx)
        s.encode(g, x, inp["k_cb"], kidx, pt=pt)
        s.encode(g, inp["v"].contiguous(), inp["v_cb"], vidx)
        torch.cuda.synchronize()
        for b in range(2):
            for h in range(2):
                rk, rv = _check_encode_slice(cfg, inp, kidx, vidx, sigma, b, h, slice(None))
                assert rk[2] == 0 and rv[2] == 0, (N, b, h, rk, rv)
