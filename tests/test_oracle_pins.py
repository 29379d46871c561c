"""Pins of the fp64 oracle against what the LoopVQ review (arXiv 2611.05304)
and plain mathematics fix.  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(rng, shape, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.bfloat16)
    return x.double().numpy()


# --------------------------------------------------------------- closed forms

def test_worked_example_counts():
    g = _gold("worked_example.json")
    D, T, K, G = g["D"], g["T"], g["K"], g["G"]
    assert ref.bits_per_element(K, G) == g["bits_per_element"]
    assert D // G == g["cq"]["indices_per_step"]
    assert ref.indices_per_token_head_cq(D, G, T) == g["cq"]["indices_total"]
    lv = g["loopvq"]
    c = G // lv["T_c"]
    assert c == lv["chunk_channels_per_step"]
    assert ref.indices_per_token_head_block(D, G, lv["T_c"]) == lv["chunks"] == lv["indices_total"]
    # T = T_c: one block, one index row, as many indices as per-step CQ
    assert (T // lv["T_c"]) * ref.indices_per_token_head_block(D, G, lv["T_c"]) == \
        ref.indices_per_token_head_cq(D, G, T)
    # one index covers its chunk's channels at every step of the block
    z = ref.joint_vectors(np.zeros((T, 1, D)), lv["T_c"], G)
    assert z.shape == (T // lv["T_c"], 1, lv["chunks"], G)


def test_bit_accounting_printed_values():
    g = _gold("bit_accounting.json")
    for case in g["cases"]:
        assert ref.bits_per_element(case["K"], case["G"]) == case["bits"]
        sb = ref.sigma_bits_per_key_element(case["H"], case["D"])
        assert round(sb, 3) == case["sigma_bits_3dp"]
        assert round(case["bits"] + sb, 3) == case["key_bits_with_sigma_3dp"]
        c = case["G"] // case["T_c"]
        per_step_idx_bytes = ref.indices_per_token_head_block(case["D"], case["G"], case["T_c"])
        assert (2 * case["D"]) / per_step_idx_bytes == case["bytes_ratio_vs_bf16"]
        assert 2 * c == case["bytes_ratio_vs_bf16"]
    # 0.5 bit is 32x smaller than bf16 (section 'terms')
    assert 16 / ref.bits_per_element(256, 16) == 32


def test_joint_layout_hand_worked():
    g = _gold("joint_layout.json")
    x = np.array(g["x_steps"], dtype=np.float64)[:, None, :]   # [T, N=1, D]
    z = ref.joint_vectors(x, g["T_c"], g["G"])
    assert np.array_equal(z[0, 0], np.array(g["joint_chunks"], dtype=np.float64))


def test_chunk_locality():
    """Changing channel d of step t changes only chunk d // c of block t // T_c."""
    rng = np.random.default_rng(1)
    T, T_c, D, G = 8, 4, 32, 16
    c = G // T_c
    x = rng.standard_normal((T, 3, D))
    z0 = ref.joint_vectors(x, T_c, G)
    for (t, j, d) in [(0, 0, 0), (5, 2, 17), (7, 1, 31), (3, 0, 4)]:
        x2 = x.copy()
        x2[t, j, d] += 1.0
        diff = np.argwhere(ref.joint_vectors(x2, T_c, G) != z0)
        assert diff.shape[0] == 1
        beta, jj, q, u = diff[0]
        assert (beta, jj, q) == (t // T_c, j, d // c)
        assert u == (d % c) * T_c + (t % T_c)


# --------------------------------------------------------------- encode

def _exact_argmin(z, cb):
    """Brute force with exact rational arithmetic; lowest index on ties."""
    best, arg = None, None
    zf = [Fraction(float(v)) for v in z]
    for r in range(cb.shape[0]):
        d = sum((zf[u] - Fraction(float(cb[r, u]))) ** 2 for u in range(len(zf)))
        if best is None or d < best:
            best, arg = d, r
    return arg


@pytest.mark.parametrize("G,T_c,K", [(4, 2, 16), (8, 4, 8), (16, 4, 16), (16, 1, 5)])
def test_argmin_brute_force(G, T_c, K):
    rng = np.random.default_rng(100 + G + K)
    c = G // T_c
    D = 4 * c
    cb = _bf16(rng, (1, K, G))
    cb[0, K - 1] = cb[0, 1]           # duplicate codeword: lowest index must win
    x = _bf16(rng, (T_c, 16, D))
    # plant exact codewords and exact midpoints (ties) in a few tokens
    for j in range(4):
        r = int(rng.integers(K))
        for m in range(T_c):
            for q in range(D // c):
                for i in range(c):
                    x[m, j, q * c + i] = cb[0, r, i * T_c + m]
    idx, ties = ref.encode(x, cb, T_c)
    z = ref.joint_vectors(x, T_c, G)
    for j in range(x.shape[1]):
        for q in range(D // c):
            assert idx[0, j, q] == _exact_argmin(z[0, j, q], cb[0])
    assert ties.max() >= 2            # the duplicate produced a recorded tie


def test_codeword_inputs_reconstruct_exactly():
    rng = np.random.default_rng(7)
    T, T_c, D, G, K = 8, 4, 128, 16, 256
    c = G // T_c
    cb = _bf16(rng, (T // T_c, K, G), 2.0)
    N = 40
    want = rng.integers(0, K, size=(T // T_c, N, D // c))
    x = np.empty((T, N, D))
    for beta in range(T // T_c):
        for m in range(T_c):
            for i in range(c):
                x[beta * T_c + m, :, i::c] = cb[beta][want[beta], i * T_c + m]
    idx, ties = ref.encode(x, cb, T_c)
    # random bf16 codewords are distinct, so the index is recovered exactly
    assert np.array_equal(idx, want)
    assert np.array_equal(ref.dequant(idx, cb, T_c, D), x)


def test_tc1_is_channel_vq_scipy():
    vq = pytest.importorskip("scipy.cluster.vq")
    rng = np.random.default_rng(3)
    T, D, G, K = 4, 64, 16, 32
    cb = _bf16(rng, (T, K, G))        # T_c = 1: one codebook per step, eq. (2)
    x = _bf16(rng, (T, 50, D))
    idx, ties = ref.encode(x, cb, 1)
    for t in range(T):
        chunks = x[t].reshape(-1, G)  # consecutive G channels
        code, _ = vq.vq(chunks, cb[t], check_finite=True)
        ok = ties[t].reshape(-1) == 1
        assert ok.mean() > 0.99
        assert np.array_equal(code[ok], idx[t].reshape(-1)[ok])


def test_encode_invariances():
    rng = np.random.default_rng(11)
    T_c, D, G, K = 4, 32, 16, 64
    cb = _bf16(rng, (1, K, G))
    x = _bf16(rng, (T_c, 30, D))
    idx, ties = ref.encode(x, cb, T_c)
    perm = rng.permutation(K)
    idx_p, _ = ref.encode(x, cb[:, perm], T_c)
    ok = ties == 1                    # row r' of the permuted book is row perm[r']
    assert np.array_equal(perm[idx_p][ok], idx[ok])
    for k in (-3, 5):
        idx_s, _ = ref.encode(x * 2.0 ** k, cb * 2.0 ** k, T_c)
        assert np.array_equal(idx_s, idx)


def test_tie_set_semantics():
    cb = np.array([[[0.0, 0.0], [2.0, 0.0], [0.0, 2.0]]])
    z = np.array([[[[1.0, 0.0]]]])            # equidistant to codewords 0 and 1
    a, ties = ref.nearest_codeword(z[0], cb[0])
    assert a[0, 0] == 0 and ties[0, 0] == 2
    assert ref.tie_set_contains(z[0], cb[0], np.array([[1]]))[0, 0]
    assert not ref.tie_set_contains(z[0], cb[0], np.array([[2]]))[0, 0]


# --------------------------------------------------------------- RoPE

def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(5)
    D, P = 128, 40
    x = rng.standard_normal((P, D))
    pos = rng.integers(0, 70000, size=P)
    y = ref.apply_rope(x, pos)
    h = D // 2
    omega = 1e4 ** (-np.arange(h) * 2.0 / D)
    zc = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * pos[:, None] * omega[None, :])
    assert np.allclose(y[:, :h], zc.real, atol=1e-12, rtol=0)
    assert np.allclose(y[:, h:], zc.imag, atol=1e-12, rtol=0)


def test_rope_closed_forms_and_group():
    D = 128
    phi = ref.rope_angles(np.array([0, 1, 100]), D)
    assert np.all(phi[0] == 0)
    assert phi[1, 0] == 1.0                          # omega_0 = 1
    assert abs(phi[2, D // 4] - 1.0) < 1e-15         # theta^(-1/2) = 1e-2
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal((2, 1, D))
    a, b = 1234, 57
    x0 = ref.apply_rope(k, [0])
    assert np.array_equal(x0, k)
    assert abs(np.linalg.norm(ref.apply_rope(k, [a])) - np.linalg.norm(k)) < 1e-12
    ab = ref.apply_rope(ref.apply_rope(k, [b]), [a])
    assert np.allclose(ab, ref.apply_rope(k, [a + b]), atol=1e-11)
    lhs = float((ref.apply_rope(q, [a]) @ ref.apply_rope(k, [b]).T)[0, 0])
    rhs = float((q @ ref.apply_rope(k, [b - a]).T)[0, 0])
    assert abs(lhs - rhs) < 1e-10
    tab = ref.rope_table(70000, D)
    assert np.allclose(tab[65540, :, 0], np.cos(65540 * 1e4 ** (-np.arange(64) / 64.0)), atol=1e-12)


# --------------------------------------------------------------- attention

def test_attention_matches_sdpa_with_sinks():
    rng = np.random.default_rng(13)
    T, T_c, D, G, K, N, n_s = 8, 4, 128, 16, 32, 25, 4
    cb_k = _bf16(rng, (2, K, G))
    cb_v = _bf16(rng, (2, K, G))
    k_idx = rng.integers(0, K, size=(2, N, D // 4))
    v_idx = rng.integers(0, K, size=(2, N, D // 4))
    sk = _bf16(rng, (T, n_s, D))
    sv = _bf16(rng, (T, n_s, D))
    kh = ref.dequant(k_idx, cb_k, T_c, D)
    vh = ref.dequant(v_idx, cb_v, T_c, D)
    h = D // 2
    omega = 1e4 ** (-np.arange(h) * 2.0 / D)
    for t in (0, 3, 6):
        q = rng.standard_normal(D)
        out, lse = ref.decode_attn_row(q, t, k_idx, v_idx, cb_k, cb_v, sk, sv, T_c)
        keys = np.concatenate([sk[t], kh[t]])
        pos = np.arange(n_s + N)
        zc = (keys[:, :h] + 1j * keys[:, h:]) * np.exp(1j * pos[:, None] * omega)
        krot = np.concatenate([zc.real, zc.imag], axis=1)
        vals = np.concatenate([sv[t], vh[t]])
        sd = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None], torch.from_numpy(krot)[None, None],
            torch.from_numpy(vals)[None, None])
        assert np.allclose(out, sd[0, 0, 0].numpy(), atol=1e-12, rtol=1e-12)
        s = krot @ q / math.sqrt(D)
        assert abs(lse - float(torch.logsumexp(torch.from_numpy(s), 0))) < 1e-12


def test_recent_window_is_the_same_softmax():
    """Section 3.4: the newest tokens stay bf16 and are attended in the same
    softmax; their positions follow the quantized tokens.  Equivalent to
    Flash-Decoding merge of the compressed part with a bf16 segment."""
    rng = np.random.default_rng(31)
    T, T_c, D, G, K, N, n_s, n_r = 4, 4, 128, 16, 32, 20, 3, 5
    cb_k, cb_v = _bf16(rng, (1, K, G)), _bf16(rng, (1, K, G))
    ki = rng.integers(0, K, size=(1, N, D // 4))
    vi = rng.integers(0, K, size=(1, N, D // 4))
    sk, sv = _bf16(rng, (T, n_s, D)), _bf16(rng, (T, n_s, D))
    rk, rv = _bf16(rng, (T, n_r, D)), _bf16(rng, (T, n_r, D))
    for t in range(T):
        q = rng.standard_normal(D)
        full = ref.decode_attn_row(q, t, ki, vi, cb_k, cb_v, sk, sv, T_c, recent_k=rk, recent_v=rv)
        base = ref.decode_attn_row(q, t, ki, vi, cb_k, cb_v, sk, sv, T_c)
        seg = ref.attention(q, ref.apply_rope(rk[t], np.arange(n_s + N, n_s + N + n_r)), rv[t])
        out, lse = ref.lse_merge([base, seg])
        assert np.allclose(full[0], out, atol=1e-12) and abs(full[1] - lse) < 1e-12
        # and equals SDPA over the explicit key sequence sinks | codes | recent
        keys = np.concatenate([sk[t], ref.dequant(ki, cb_k, T_c, D)[t], rk[t]])
        pos = np.arange(keys.shape[0])
        vals = np.concatenate([sv[t], ref.dequant(vi, cb_v, T_c, D)[t], rv[t]])
        sd = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None], torch.from_numpy(ref.apply_rope(keys, pos))[None, None],
            torch.from_numpy(vals)[None, None])
        assert np.allclose(full[0], sd[0, 0, 0].numpy(), atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(17)
    D, P = 16, 9
    k = rng.standard_normal((P, D))
    v = rng.standard_normal((P, D))
    out, lse = ref.attention(np.zeros(D), k, v)
    assert np.allclose(out, v.mean(0), atol=1e-14)
    assert abs(lse - math.log(P)) < 1e-14
    out, lse = ref.attention(rng.standard_normal(D), k[:1], v[:1])
    assert np.allclose(out, v[0], atol=1e-15)
    q = 200.0 * k[4] / np.linalg.norm(k[4])
    kk = k / np.linalg.norm(k, axis=1, keepdims=True)
    out, _ = ref.attention(q, kk * math.sqrt(D), v)
    assert np.allclose(out, v[4], atol=1e-6)


def test_lse_merge_split_invariance():
    rng = np.random.default_rng(19)
    D, P = 32, 50
    q, k, v = rng.standard_normal(D), rng.standard_normal((P, D)), rng.standard_normal((P, D))
    full = ref.attention(q, k, v)
    for cuts in ([10], [1, 30], [7, 8, 40]):
        bounds = [0] + cuts + [P]
        parts = [ref.attention(q, k[a:b], v[a:b]) for a, b in zip(bounds, bounds[1:])]
        out, lse = ref.lse_merge(parts)
        assert np.allclose(out, full[0], atol=1e-13) and abs(lse - full[1]) < 1e-13


# --------------------------------------------------------------- pre-transform

def test_fp16_round():
    assert ref.fp16_round(1.0 + 2.0 ** -11) == 1.0               # tie to even
    assert ref.fp16_round(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9
    assert ref.fp16_round(65504.0) == 65504.0


def test_tasq_sigma_and_identity():
    rng = np.random.default_rng(23)
    H, T, N, D = 3, 4, 6, 8
    k = rng.standard_normal((H, T, N, D))
    s = ref.tasq_sigma(k)
    assert s.shape == (N, T)
    assert np.allclose(ref.tasq_sigma(np.full((H, T, N, D), -2.5)), 2.5)
    assert np.allclose(ref.tasq_sigma(3.0 * k), 3.0 * s)
    manual = math.sqrt(sum(k[h, 1, 2, d] ** 2 for h in range(H) for d in range(D)) / (H * D))
    assert abs(s[2, 1] - manual) < 1e-14
    w = np.exp(0.3 * rng.standard_normal(D))
    perm = rng.permutation(D)
    sb = ref.fp16_round(s[:, 0])
    z = ref.tasq_forward(k[0, 0], w, perm, sb)
    assert np.allclose(ref.tasq_inverse(z, w, perm, sb), k[0, 0], rtol=1e-14, atol=0)
    # identity transform gives the plain encode
    cb = _bf16(rng, (1, 16, 8))
    x = _bf16(rng, (4, N, 8))
    a0, _ = ref.encode(x, cb, 4)
    a1, _ = ref.encode_tasq(x, cb, 4, np.ones(8), np.arange(8), np.ones((N, 4)))
    assert np.array_equal(a0, a1)


def test_tasq_forward_hand_worked():
    g = _gold("tasq_forward.json")
    z = ref.tasq_forward(np.array([g["k"]], dtype=np.float64), np.array(g["w"]),
                         np.array(g["perm"]), np.array([g["sigma"]]))
    assert np.array_equal(z[0], np.array(g["z"], dtype=np.float64))


def test_tasq_codeword_inputs_roundtrip():
    rng = np.random.default_rng(29)
    T_c, D, G, K, N = 4, 32, 16, 64, 10
    c = G // T_c
    cb = _bf16(rng, (1, K, G))
    want = rng.integers(0, K, size=(1, N, D // c))
    zt = ref.dequant(want, cb, T_c, D)                       # transformed-space keys
    w = np.exp(0.3 * rng.standard_normal(D))
    perm = rng.permutation(D)
    sb = ref.fp16_round(np.exp(rng.standard_normal((N, T_c))))
    k = np.stack([ref.tasq_inverse(zt[t], w, perm, sb[:, t]) for t in range(T_c)])
    idx, _ = ref.encode_tasq(k, cb, T_c, w, perm, sb)
    assert np.array_equal(idx, want)
    sink_k = np.zeros((T_c, 0, D))
    for t in range(T_c):
        q = rng.standard_normal(D)
        o1, l1 = ref.decode_attn_row(q, t, idx, idx, cb, cb, sink_k, sink_k, T_c,
                                     tasq=(w, perm, sb))
        o2, l2 = ref.attention(q, ref.apply_rope(k[t], np.arange(N)), ref.dequant(idx, cb, T_c, D)[t])
        assert np.allclose(o1, o2, atol=1e-12) and abs(l1 - l2) < 1e-12


# --------------------------------------------------------------- Fig. 2c direction

def test_loop_axis_lowers_nmse():
    """Section 1.2 / Fig. 2c: grouping along the loop axis lowers k-means
    reconstruction error at fixed bits and codebook count (direction only)."""
    from synth import codebooks as cbmod
    from synth.configs import config_by_index
    from synth.generator import gen_kv_layer
    import dataclasses
    cfg = dataclasses.replace(config_by_index(1), N=384)
    x = gen_kv_layer(cfg, 0, "k", "cpu")[0, 0].double().numpy()      # [T, N, D]
    train, test = x[:, :256], x[:, 256:]
    g = torch.Generator().manual_seed(5)
    K, G, T = 256, 16, cfg.T

    def fit(vecs):
        return cbmod._kmeans(torch.from_numpy(vecs)[None], K, 25, g)[0].numpy()

    # loop-axis: T_c = 4, c = 4
    zl = ref.joint_vectors(train, 4, G)[0].reshape(-1, G)
    cbl = fit(zl)[None]
    il, _ = ref.encode(test, cbl, 4)
    e_loop = ref.nmse(test, ref.dequant(il, cbl, 4, cfg.D))
    # per-step grouping: 16 consecutive channels of one step; one shared codebook
    zs = np.concatenate([ref.joint_vectors(train[t:t + 1], 1, G)[0].reshape(-1, G) for t in range(T)])
    cbs = fit(zs)
    is_, _ = ref.encode(test, np.repeat(cbs[None], T, 0), 1)
    e_shared = ref.nmse(test, ref.dequant(is_, np.repeat(cbs[None], T, 0), 1, cfg.D))
    # per-step codebooks (channel VQ baseline, 4 codebooks)
    cbp = np.stack([fit(ref.joint_vectors(train[t:t + 1], 1, G)[0].reshape(-1, G)) for t in range(T)])
    ip, _ = ref.encode(test, cbp, 1)
    e_cq = ref.nmse(test, ref.dequant(ip, cbp, 1, cfg.D))
    assert e_loop < e_shared and e_loop < e_cq


# --------------------------------------------------------------- NMSE (Fig. 2c's measure)

def test_nmse_closed_forms():
    """Section 1.2 / Fig. 2c reports reconstruction error as NMSE: squared
    error over squared signal, pooled over all tokens, steps and channels."""
    # hand-worked: one channel of (3, 4) lost -> 9 / 25
    assert ref.nmse(np.array([3.0, 4.0]), np.array([0.0, 4.0])) == 9.0 / 25.0
    # pooled ratio, not a mean of per-row ratios: (0 + 1) / (25 + 1)
    x = np.array([[3.0, 4.0], [1.0, 0.0]])
    assert ref.nmse(x, np.array([[3.0, 4.0], [0.0, 0.0]])) == 1.0 / 26.0
    rng = np.random.default_rng(21)
    x = rng.standard_normal((4, 7, 16)) + 0.5
    # reconstructing nothing leaves all the energy
    assert ref.nmse(x, np.zeros_like(x)) == pytest.approx(1.0, rel=1e-15)
    # shrinking by (1 - a) leaves a^2 of it
    for a in (0.5, 0.125, 0.3):
        assert ref.nmse(x, (1.0 - a) * x) == pytest.approx(a * a, rel=1e-12)
    # uncentred: a constant signal reconstructed at half its level keeps 1/4
    assert ref.nmse(np.full(8, 2.0), np.full(8, 1.0)) == 0.25
    # one-entry codebook at the mean: error / energy = variance / second moment
    v = rng.standard_normal(5000) * 2.0 + 1.0
    assert ref.nmse(v, np.full_like(v, v.mean())) == pytest.approx(v.var() / np.mean(v * v), rel=1e-12)
