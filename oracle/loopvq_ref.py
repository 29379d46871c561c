"""Plain fp64 definitions of LoopVQ encode and decode attention.

TEST INFRASTRUCTURE: imported only by tests, smoke() and the benchmark's
CPU-baseline leg.

Source: the LoopVQ review page (jaehun.me, "paper-2611-05304v1", a review of
arXiv 2611.05304).  Sections cited below are that page's.

Readings taken where the page is silent (each is listed with its reason in the
design notes of the repository):
  * chunk q holds the c consecutive channels [q*c, q*c + c);
  * joint coordinate i*T_c + m is channel q*c + i at block step m;
  * one codebook per (layer, kv-head, K or V, block), shared by all chunks;
  * argmin ties go to the lowest index; the tie set is every r with
    d_r <= (1 + 1e-6) * d_min;
  * RoPE is rotate-half over pairs (d, d + D/2), angle pos * theta^(-2d/D),
    computed in fp64; keys (sinks included) are stored pre-RoPE, queries are
    given already rotated; sink s sits at position s, quantized token j at
    position n_s + j;
  * softmax scale 1/sqrt(D), natural exp, no mask beyond the cache itself;
  * GQA: q-head hq reads kv-head floor(hq * H_kv / H_q);
  * pre-transform (appendix B, eq. 10): sigma = RMS over the layer's H_kv*D
    raw key channels of one (token, step), rounded to fp16; the transformed
    key is z[d'] = (w[p(d')] * k[p(d')]) / sigma, p the channel permutation.
"""
import math
import numpy as np

TIE_REL = 1e-6


# ----------------------------------------------------------------------------
# bit accounting (section "terms": vector quantization; section 3.1; 3.3)
# ----------------------------------------------------------------------------

def bits_per_element(K: int, G: int) -> float:
    """b/G bits per cached element for a K = 2^b entry codebook over G-vectors."""
    b = int(round(math.log2(K)))
    assert 2 ** b == K
    return b / G


def sigma_bits_per_key_element(H: int, D: int) -> float:
    """An fp16 per-token scale shared by H heads of D channels costs 16/(H*D) bits."""
    return 16.0 / (H * D)


def indices_per_token_head_block(D: int, G: int, T_c: int) -> int:
    """One index per chunk of c = G/T_c channels: D/c indices per (token, head, block)."""
    c = G // T_c
    assert c * T_c == G and D % c == 0
    return D // c


def indices_per_token_head_cq(D: int, G: int, T: int) -> int:
    """Per-step channel VQ (eq. 2): D/G indices per step, T steps."""
    assert D % G == 0
    return T * (D // G)


# ----------------------------------------------------------------------------
# encode: eq. (2) nearest codeword; eq. (4) joint loop-axis vector
# ----------------------------------------------------------------------------

def joint_vectors(x: np.ndarray, T_c: int, G: int) -> np.ndarray:
    """Loop-axis joint vectors (section 3.1, eq. 4).

    x: [..., T, N, D] -> z: [..., n_blk, N, D/c, G] with
    z[..., beta, j, q, i*T_c + m] = x[..., beta*T_c + m, j, q*c + i].
    """
    x = np.asarray(x, dtype=np.float64)
    *lead, T, N, D = x.shape
    c = G // T_c
    n_blk = T // T_c
    z = np.empty(tuple(lead) + (n_blk, N, D // c, G), dtype=np.float64)
    for beta in range(n_blk):
        for m in range(T_c):
            step = x[..., beta * T_c + m, :, :]            # [..., N, D]
            for i in range(c):
                z[..., beta, :, :, i * T_c + m] = step[..., i::c]
    return z


def squared_distances(z: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """d_r = sum_u (z[u] - e_r[u])^2, direct form, fp64.  z [..., G], cb [K, G] -> [..., K]."""
    z = np.asarray(z, dtype=np.float64)
    cb = np.asarray(cb, dtype=np.float64)
    diff = z[..., None, :] - cb
    return np.einsum("...kg,...kg->...k", diff, diff)


def nearest_codeword(z: np.ndarray, cb: np.ndarray):
    """Eq. (2): a(z) = argmin_r ||z - e_r||^2, lowest index on exact ties.

    Returns (a, tie_count): tie_count = |{r : d_r <= (1 + 1e-6) d_min}|.
    """
    d = squared_distances(z, cb)
    a = np.argmin(d, axis=-1)          # numpy returns the first minimum
    dmin = np.take_along_axis(d, a[..., None], axis=-1)
    ties = (d <= dmin * (1.0 + TIE_REL)).sum(axis=-1)
    return a, ties


def tie_set_contains(z: np.ndarray, cb: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """True where idx lies in the tie set A(z)."""
    d = squared_distances(z, cb)
    dmin = d.min(axis=-1, keepdims=True)
    di = np.take_along_axis(d, np.asarray(idx, dtype=np.int64)[..., None], axis=-1)
    return (di <= dmin * (1.0 + TIE_REL))[..., 0]


def encode(x: np.ndarray, cb: np.ndarray, T_c: int):
    """Encode one (batch, kv-head) slice.

    x: [T, N, D] per-step cache; cb: [n_blk, K, G] codebooks.
    Returns (idx [n_blk, N, D/c] int64, ties [n_blk, N, D/c]).
    """
    G = cb.shape[-1]
    z = joint_vectors(x, T_c, G)                         # [n_blk, N, D/c, G]
    idx = np.empty(z.shape[:-1], dtype=np.int64)
    ties = np.empty(z.shape[:-1], dtype=np.int64)
    for beta in range(z.shape[0]):
        idx[beta], ties[beta] = nearest_codeword(z[beta], cb[beta])
    return idx, ties


# ----------------------------------------------------------------------------
# dequant: eq. (5), step t reads its slice B_t of the shared codeword
# ----------------------------------------------------------------------------

def dequant(idx: np.ndarray, cb: np.ndarray, T_c: int, D: int) -> np.ndarray:
    """idx [n_blk, N, D/c], cb [n_blk, K, G] -> x_hat [T, N, D] (fp64).

    x_hat[beta*T_c + m, j, q*c + i] = cb[beta, idx[beta, j, q], i*T_c + m].
    """
    n_blk, N, n_chunk = idx.shape
    G = cb.shape[-1]
    c = G // T_c
    assert n_chunk * c == D
    out = np.empty((n_blk * T_c, N, D), dtype=np.float64)
    for beta in range(n_blk):
        e = np.asarray(cb[beta], dtype=np.float64)[idx[beta]]     # [N, D/c, G]
        for m in range(T_c):
            for i in range(c):
                out[beta * T_c + m, :, i::c] = e[:, :, i * T_c + m]
    return out


# ----------------------------------------------------------------------------
# RoPE after dequant (section "terms": RoPE; section 3.4 step 3)
# ----------------------------------------------------------------------------

def rope_angles(positions: np.ndarray, D: int, theta: float = 1.0e4) -> np.ndarray:
    """phi[p, d] = pos_p * theta^(-2d/D), d < D/2, in fp64."""
    pos = np.asarray(positions, dtype=np.float64)
    d = np.arange(D // 2, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * d / D)
    return pos[:, None] * omega[None, :]


def rope_table(n_pos: int, D: int, theta: float = 1.0e4) -> np.ndarray:
    """[n_pos, D/2, 2] (cos, sin) in fp64."""
    phi = rope_angles(np.arange(n_pos), D, theta)
    return np.stack([np.cos(phi), np.sin(phi)], axis=-1)


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float = 1.0e4) -> np.ndarray:
    """Rotate-half RoPE on pairs (d, d + D/2).  x [..., P, D], positions [P]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    phi = rope_angles(positions, D, theta)
    cs, sn = np.cos(phi), np.sin(phi)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * cs - b * sn, b * cs + a * sn], axis=-1)


# ----------------------------------------------------------------------------
# attention with sinks, online-softmax result in closed form (section 3.4)
# ----------------------------------------------------------------------------

def attention(q: np.ndarray, k_rot: np.ndarray, v: np.ndarray):
    """Softmax attention of one query over P keys.  q [D], k_rot [P, D], v [P, D].

    Returns (out [D], lse) with scale 1/sqrt(D) and natural log-sum-exp.
    """
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[-1]
    s = (np.asarray(k_rot, dtype=np.float64) @ q) / math.sqrt(D)
    mu = s.max()
    e = np.exp(s - mu)
    Z = e.sum()
    out = (e[:, None] * np.asarray(v, dtype=np.float64)).sum(axis=0) / Z
    return out, mu + math.log(Z)


def lse_merge(parts):
    """Flash-Decoding combine of (out, lse) partials over disjoint key sets."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    mu = lses.max()
    w = np.exp(lses - mu)
    out = sum(wi * np.asarray(p[0], dtype=np.float64) for wi, p in zip(w, parts)) / w.sum()
    return out, mu + math.log(w.sum())


def decode_attn_row(q_t: np.ndarray, t: int, k_idx, v_idx, k_cb, v_cb,
                    sink_k, sink_v, T_c: int, theta: float = 1.0e4,
                    n_tokens=None, tasq=None, recent_k=None, recent_v=None):
    """Decode attention of one query row (one batch entry, one q-head, step t).

    q_t: [D] post-RoPE query.  k_idx, v_idx: [n_blk, N, D/c] for the kv-head.
    k_cb, v_cb: [n_blk, K, G].  sink_k, sink_v: [T, n_s, D] pre-RoPE bf16 values.
    n_tokens: quantized tokens attended (default all N).
    tasq: None or (w [D], perm [D], sigma [N, T]) for keys of this kv-head.
    recent_k, recent_v: None or [T, n_r, D] pre-RoPE bf16 values of the recent
    window (section 3.4 step 1: the newest tokens stay bf16), at positions
    n_s + n_tokens .. n_s + n_tokens + n_r - 1.
    Returns (out [D], lse).
    """
    D = q_t.shape[-1]
    beta, m = divmod(t, T_c)
    N = k_idx.shape[1] if n_tokens is None else n_tokens
    n_s = sink_k.shape[1]
    kq = _dequant_step(k_idx[beta, :N], k_cb[beta], T_c, m, D)      # [N, D]
    vq = _dequant_step(v_idx[beta, :N], v_cb[beta], T_c, m, D)
    if tasq is not None:
        w, perm, sigma = tasq
        kq = tasq_inverse(kq, w, perm, sigma[:N, t])
    ks = [np.asarray(sink_k[t], dtype=np.float64), kq]
    vs = [np.asarray(sink_v[t], dtype=np.float64), vq]
    if recent_k is not None:
        ks.append(np.asarray(recent_k[t], dtype=np.float64))
        vs.append(np.asarray(recent_v[t], dtype=np.float64))
    keys = np.concatenate(ks, axis=0)
    vals = np.concatenate(vs, axis=0)
    pos = np.arange(keys.shape[0])
    return attention(q_t, apply_rope(keys, pos, theta), vals)


def _dequant_step(idx_blk, cb_blk, T_c, m, D):
    """Step m of one block: x_hat[j, q*c + i] = cb[idx[j, q], i*T_c + m]."""
    G = cb_blk.shape[-1]
    c = G // T_c
    e = np.asarray(cb_blk, dtype=np.float64)[idx_blk]          # [N, D/c, G]
    sl = e[:, :, m::T_c]                                        # [N, D/c, c]
    return sl.reshape(idx_blk.shape[0], D)


# ----------------------------------------------------------------------------
# channel pre-transform (section 3.3, appendix B eq. 10), keys only
# ----------------------------------------------------------------------------

def fp16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest fp16 value (ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def tasq_sigma(k_layer: np.ndarray) -> np.ndarray:
    """k_layer [H, T, N, D] (one batch entry) -> sigma [N, T] in fp64 (before fp16 rounding).

    sigma = sqrt(mean over the H*D raw key channels of k^2) for each (token, step).
    """
    k = np.asarray(k_layer, dtype=np.float64)
    return np.sqrt(np.mean(k * k, axis=(0, 3))).T


def tasq_forward(k: np.ndarray, w: np.ndarray, perm: np.ndarray, sigma_bar: np.ndarray) -> np.ndarray:
    """z[..., d'] = (w[p(d')] * k[..., p(d')]) / sigma_bar.  k [..., P, D], sigma_bar [P]."""
    k = np.asarray(k, dtype=np.float64)
    p = np.asarray(perm, dtype=np.int64)
    num = np.asarray(w, dtype=np.float64)[p] * k[..., p]
    return num / np.asarray(sigma_bar, dtype=np.float64)[..., :, None]


def tasq_inverse(z: np.ndarray, w: np.ndarray, perm: np.ndarray, sigma_bar: np.ndarray) -> np.ndarray:
    """Inverse of tasq_forward: k[..., p(d')] = z[..., d'] * sigma_bar / w[p(d')]."""
    z = np.asarray(z, dtype=np.float64)
    p = np.asarray(perm, dtype=np.int64)
    out = np.empty_like(z)
    out[..., p] = z * np.asarray(sigma_bar, dtype=np.float64)[..., :, None] / np.asarray(w, dtype=np.float64)[p]
    return out


def encode_tasq(k_head: np.ndarray, cb: np.ndarray, T_c: int, w, perm, sigma_bar):
    """Pre-transformed key encode of one (batch, kv-head): k_head [T, N, D], sigma_bar [N, T]."""
    T = k_head.shape[0]
    zt = np.stack([tasq_forward(k_head[t], w, perm, sigma_bar[:, t]) for t in range(T)])
    return encode(zt, cb, T_c)


# ----------------------------------------------------------------------------
# reconstruction error (section 1.2, Fig. 2c)
# ----------------------------------------------------------------------------

def nmse(x: np.ndarray, x_hat: np.ndarray) -> float:
    """sum ||x - x_hat||^2 / sum ||x||^2 (uncentred)."""
    x = np.asarray(x, dtype=np.float64)
    e = x - np.asarray(x_hat, dtype=np.float64)
    return float((e * e).sum() / (x * x).sum())
