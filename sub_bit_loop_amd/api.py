"""Thin torch-facing binding of the LoopVQ C ABI (argument marshalling only).

Every tensor must already live on the current HIP device with the documented
dtype and layout; the calls are enqueued on torch's current stream.
"""
import ctypes

import torch

from . import _lib
from ._lib import Geom, PreTransform, check


def geom(D, T, T_c, G, K, n_kv_heads, n_q_heads, rope_theta=1.0e4) -> Geom:
    return Geom(D, T, T_c, G, K, n_kv_heads, n_q_heads, rope_theta)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)


def _shape(t, want, name):
    """want: a tuple of ints or None (any size); raises ValueError on mismatch."""
    if t.dim() != len(want) or any(w is not None and w != d for w, d in zip(want, t.shape)):
        shown = tuple("*" if w is None else w for w in want)
        raise ValueError("%s must have shape %s (got %s)" % (name, shown, tuple(t.shape)))


def _dims(g):
    """(n_blk, chunks per token) of a geometry."""
    return g.T // g.T_c, g.D // (g.G // g.T_c)


def _check_pt(g, pt, B, n_tok):
    """The pre-transform's tensors against the geometry (B batch entries,
    n_tok = the highest token position written or read)."""
    if pt is None:
        return
    w, perm, sigma = pt._keep
    _shape(w, (g.n_kv_heads, g.D), "w")
    _shape(perm, (g.n_kv_heads, g.D), "perm")
    for t, n in ((w, "w"), (perm, "perm"), (sigma, "sigma")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    if sigma.dim() != 3 or sigma.shape[0] < B or sigma.shape[1] < n_tok or sigma.shape[2] != g.T:
        raise ValueError("sigma must be [>=%d][>=%d][%d] (got %s)" % (B, n_tok, g.T, tuple(sigma.shape)))


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def pretransform(w, perm, sigma):
    """Keys' channel pre-transform: w fp32 [H][D], perm int16 [H][D], sigma fp16 [B][N_cap][T]."""
    _need(w, torch.float32, "w")
    _need(perm, torch.int16, "perm")
    _need(sigma, torch.float16, "sigma")
    pt = PreTransform(w.data_ptr(), perm.data_ptr(), sigma.data_ptr(), sigma.shape[1])
    pt._keep = (w, perm, sigma)
    return pt


def encode(g: Geom, x, codebook, idx, tok0=0, pt=None, stream=None):
    """x bf16 [B][H][T][N][D] (any strides with D contiguous), codebook bf16
    [H][n_blk][K][G], idx uint8 [B][H][n_blk][N_cap][D/c] (written)."""
    _need(x, torch.bfloat16, "x")
    _need(codebook, torch.bfloat16, "codebook")
    _need(idx, torch.uint8, "idx")
    if x.dim() != 5 or x.stride(4) != 1:
        raise ValueError("x must be [B][H][T][N][D] with contiguous rows")
    if not codebook.is_contiguous() or not idx.is_contiguous():
        raise ValueError("codebook and idx must be contiguous")
    B, _, _, N, _ = x.shape
    n_blk, cpt = _dims(g)
    _shape(x, (B, g.n_kv_heads, g.T, N, g.D), "x")
    _shape(codebook, (g.n_kv_heads, n_blk, g.K, g.G), "codebook")
    _shape(idx, (B, g.n_kv_heads, n_blk, None, cpt), "idx")
    if idx.shape[3] < tok0 + N:
        raise ValueError("idx holds %d tokens, tok0 + N = %d" % (idx.shape[3], tok0 + N))
    _check_pt(g, pt, B, tok0 + N)
    strides = (ctypes.c_int64 * 4)(*[x.stride(i) for i in range(4)])
    st = _lib.lib().loopvq_encode(ctypes.byref(g), _ptr(x), strides, _ptr(codebook), B, N, tok0,
                                  _ptr(idx), idx.shape[3], ctypes.byref(pt) if pt is not None else None,
                                  _stream(stream))
    check(st)
    return idx


def tasq_covariance(g: Geom, x, w, sigma, mean=None, cov=None, stream=None):
    """Mean and covariance (fp64) of the block-stacked scaled keys w*k/sigma for
    the pre-transform's permutation.  x bf16 [B][H][T][N][D] raw keys (rows
    contiguous), w fp32 [H][D], sigma fp16 [B][N_cap][T] (written).
    Returns (mean [H][n_blk][T_c*D], cov [H][n_blk][T_c*D][T_c*D])."""
    _need(x, torch.bfloat16, "x")
    _need(w, torch.float32, "w")
    _need(sigma, torch.float16, "sigma")
    if x.dim() != 5 or x.stride(4) != 1:
        raise ValueError("x must be [B][H][T][N][D] with contiguous rows")
    B, H, T, N, D = x.shape
    _shape(x, (B, g.n_kv_heads, g.T, N, g.D), "x")
    _shape(w, (g.n_kv_heads, g.D), "w")
    if not w.is_contiguous() or not sigma.is_contiguous():
        raise ValueError("w and sigma must be contiguous")
    if sigma.dim() != 3 or sigma.shape[0] < B or sigma.shape[1] < N or sigma.shape[2] != g.T:
        raise ValueError("sigma must be [>=%d][>=%d][%d] (got %s)" % (B, N, g.T, tuple(sigma.shape)))
    F = g.T_c * g.D
    n_blk = g.T // g.T_c
    if mean is None:
        mean = torch.empty((H, n_blk, F), dtype=torch.float64, device=x.device)
    if cov is None:
        cov = torch.empty((H, n_blk, F, F), dtype=torch.float64, device=x.device)
    _need(mean, torch.float64, "mean")
    _need(cov, torch.float64, "cov")
    _shape(mean, (H, n_blk, F), "mean")
    _shape(cov, (H, n_blk, F, F), "cov")
    if not mean.is_contiguous() or not cov.is_contiguous():
        raise ValueError("mean and cov must be contiguous")
    strides = (ctypes.c_int64 * 4)(*[x.stride(i) for i in range(4)])
    check(_lib.lib().loopvq_tasq_covariance(ctypes.byref(g), _ptr(x), strides, B, N, _ptr(w), _ptr(sigma),
                                            sigma.shape[1], _ptr(mean), _ptr(cov), _stream(stream)))
    return mean, cov


def tasq_pair_permutation(cov_host, T_c, D, c):
    """Channel permutation (int16 [D], host) from one block's covariance
    (fp64 [T_c*D][T_c*D], host tensor)."""
    if not isinstance(cov_host, torch.Tensor) or cov_host.dtype != torch.float64 or cov_host.device.type != "cpu":
        raise TypeError("cov_host must be a host float64 tensor")
    cov_host = cov_host.contiguous()
    perm = torch.empty(D, dtype=torch.int16)
    check(_lib.lib().loopvq_tasq_pair_permutation(ctypes.c_void_p(cov_host.data_ptr()), T_c, D, c,
                                                  ctypes.c_void_p(perm.data_ptr())))
    return perm


def kmeans_accumulate(g: Geom, x, idx, sums, wsum, weight=None, pt=None, stream=None):
    """Adds omega*z and omega of every joint vector of x into its codeword's
    sums fp64 [H][n_blk][K][G] and wsum fp64 [H][n_blk][K].  x bf16
    [B][H][T][N][D] (rows contiguous), idx uint8 from encode(x),
    weight fp32 [B][H][n_blk][N][D/c] or None."""
    _need(x, torch.bfloat16, "x")
    _need(idx, torch.uint8, "idx")
    _need(sums, torch.float64, "sums")
    _need(wsum, torch.float64, "wsum")
    if weight is not None:
        _need(weight, torch.float32, "weight")
        if not weight.is_contiguous():
            raise ValueError("weight must be contiguous")
    if x.dim() != 5 or x.stride(4) != 1:
        raise ValueError("x must be [B][H][T][N][D] with contiguous rows")
    for t, n in ((idx, "idx"), (sums, "sums"), (wsum, "wsum")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    B, _, _, N, _ = x.shape
    n_blk, cpt = _dims(g)
    _shape(x, (B, g.n_kv_heads, g.T, N, g.D), "x")
    _shape(idx, (B, g.n_kv_heads, n_blk, None, cpt), "idx")
    if idx.shape[3] < N:
        raise ValueError("idx holds %d tokens, x has %d" % (idx.shape[3], N))
    _shape(sums, (g.n_kv_heads, n_blk, g.K, g.G), "sums")
    _shape(wsum, (g.n_kv_heads, n_blk, g.K), "wsum")
    if weight is not None:
        _shape(weight, (B, g.n_kv_heads, n_blk, N, cpt), "weight")
    _check_pt(g, pt, B, N)
    strides = (ctypes.c_int64 * 4)(*[x.stride(i) for i in range(4)])
    check(_lib.lib().loopvq_kmeans_accumulate(ctypes.byref(g), _ptr(x), strides, B, N, _ptr(idx), idx.shape[3],
                                              _ptr(weight), ctypes.byref(pt) if pt is not None else None,
                                              _ptr(sums), _ptr(wsum), _stream(stream)))


def kmeans_finalize(g: Geom, sums, wsum, codebook, stream=None):
    """codebook bf16 [H][n_blk][K][G] <- bf16(sums / wsum) where wsum > 0."""
    _need(sums, torch.float64, "sums")
    _need(wsum, torch.float64, "wsum")
    _need(codebook, torch.bfloat16, "codebook")
    for t, n in ((sums, "sums"), (wsum, "wsum"), (codebook, "codebook")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    n_blk, _ = _dims(g)
    _shape(sums, (g.n_kv_heads, n_blk, g.K, g.G), "sums")
    _shape(wsum, (g.n_kv_heads, n_blk, g.K), "wsum")
    _shape(codebook, (g.n_kv_heads, n_blk, g.K, g.G), "codebook")
    check(_lib.lib().loopvq_kmeans_finalize(ctypes.byref(g), _ptr(sums), _ptr(wsum), _ptr(codebook),
                                            _stream(stream)))
    return codebook


def rope_table(n_pos, D=128, theta=1.0e4, device="cuda", stream=None):
    """fp16 [n_pos][D/8][8]: per 4 frequencies, their cosines then sines."""
    t = torch.empty((n_pos, D // 8, 8), dtype=torch.float16, device=device)
    check(_lib.lib().loopvq_rope_table(theta, D, n_pos, _ptr(t), _stream(stream)))
    return t


def decode_workspace_bytes(g: Geom, B, N, step0, n_steps):
    out = ctypes.c_size_t(0)
    check(_lib.lib().loopvq_decode_attn_workspace(ctypes.byref(g), B, N, step0, n_steps, ctypes.byref(out)))
    return out.value


def decode_attn(g: Geom, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, N=None, step0=0,
                seq_len=None, pt=None, out=None, lse=None, workspace=None, stream=None,
                recent_k=None, recent_v=None, n_r=None):
    """q bf16 [B][Hq][n_steps][D] (post-RoPE); k_idx/v_idx uint8 [B][H][n_blk][N_cap][D/c];
    k_cb/v_cb bf16 [H][n_blk][K][G]; sinks bf16 [B][H][T][n_s][D] or None;
    recent window bf16 [B][H][T][R_cap][D] or None (first n_r tokens attended);
    rope fp16 table from rope_table().  Returns (out fp32 [B][Hq][n_steps][D], lse fp32 [B][Hq][n_steps])."""
    return _decode(g, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, N, step0, seq_len, pt, out, lse,
                   workspace, stream, recent_k, recent_v, n_r, False)


def decode_attn_noalloc(g: Geom, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, N=None, step0=0,
                        seq_len=None, pt=None, out=None, lse=None, stream=None, recent_k=None, recent_v=None,
                        n_r=None):
    """decode_attn without a workspace (loopvq_decode_attn_noalloc: the split
    partials live in the library's static per-GPU array).  out and lse are
    allocated here when not given; pass them to keep the call allocation-free."""
    return _decode(g, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, N, step0, seq_len, pt, out, lse,
                   None, stream, recent_k, recent_v, n_r, True)


def _decode(g, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, N, step0, seq_len, pt, out, lse, workspace,
            stream, recent_k, recent_v, n_r, noalloc):
    _need(q, torch.bfloat16, "q")
    _need(k_idx, torch.uint8, "k_idx")
    _need(v_idx, torch.uint8, "v_idx")
    _need(k_cb, torch.bfloat16, "k_cb")
    _need(v_cb, torch.bfloat16, "v_cb")
    _need(rope, torch.float16, "rope")
    for t, n in ((q, "q"), (k_idx, "k_idx"), (v_idx, "v_idx"), (k_cb, "k_cb"), (v_cb, "v_cb"), (rope, "rope")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    B, Hq, n_steps, D = q.shape
    n_blk, cpt = _dims(g)
    _shape(q, (B, g.n_q_heads, n_steps, g.D), "q")
    _shape(k_idx, (B, g.n_kv_heads, n_blk, None, cpt), "k_idx")
    _shape(v_idx, tuple(k_idx.shape), "v_idx")
    _shape(k_cb, (g.n_kv_heads, n_blk, g.K, g.G), "k_cb")
    _shape(v_cb, (g.n_kv_heads, n_blk, g.K, g.G), "v_cb")
    _shape(rope, (None, g.D // 8, 8), "rope")
    N_cap = k_idx.shape[3]
    N = N_cap if N is None else N
    n_s = 0
    if (sink_k is None) != (sink_v is None):
        raise ValueError("sink_k and sink_v must both be given or both be None")
    if sink_k is not None:
        _need(sink_k, torch.bfloat16, "sink_k")
        _need(sink_v, torch.bfloat16, "sink_v")
        n_s = sink_k.shape[3]
        _shape(sink_k, (B, g.n_kv_heads, g.T, n_s, g.D), "sink_k")
        _shape(sink_v, (B, g.n_kv_heads, g.T, n_s, g.D), "sink_v")
        if not sink_k.is_contiguous() or not sink_v.is_contiguous():
            raise ValueError("sink_k and sink_v must be contiguous")
    if seq_len is not None:
        _need(seq_len, torch.int32, "seq_len")
        _shape(seq_len, (B,), "seq_len")
        if not seq_len.is_contiguous():
            raise ValueError("seq_len must be contiguous")
    R_cap = 0
    if (recent_k is None) != (recent_v is None):
        raise ValueError("recent_k and recent_v must both be given or both be None")
    if recent_k is not None:
        _need(recent_k, torch.bfloat16, "recent_k")
        _need(recent_v, torch.bfloat16, "recent_v")
        R_cap = recent_k.shape[3]
        _shape(recent_k, (B, g.n_kv_heads, g.T, R_cap, g.D), "recent_k")
        _shape(recent_v, (B, g.n_kv_heads, g.T, R_cap, g.D), "recent_v")
        if not recent_k.is_contiguous() or not recent_v.is_contiguous():
            raise ValueError("recent_k and recent_v must be contiguous")
    n_r = R_cap if n_r is None else n_r
    _check_pt(g, pt, B, N)
    if out is None:
        out = torch.empty((B, Hq, n_steps, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, n_steps), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    _need(lse, torch.float32, "lse")
    _shape(out, (B, Hq, n_steps, D), "out")
    _shape(lse, (B, Hq, n_steps), "lse")
    if not out.is_contiguous() or not lse.is_contiguous():
        raise ValueError("out and lse must be contiguous")
    if noalloc:
        st = _lib.lib().loopvq_decode_attn_noalloc(
            ctypes.byref(g), _ptr(q), step0, n_steps, _ptr(k_idx), _ptr(v_idx), N_cap, _ptr(k_cb), _ptr(v_cb),
            _ptr(sink_k), _ptr(sink_v), n_s, _ptr(recent_k), _ptr(recent_v), n_r, R_cap, B, N, _ptr(seq_len),
            ctypes.byref(pt) if pt is not None else None,
            _ptr(rope), rope.shape[0], _ptr(out), _ptr(lse), _stream(stream))
        check(st)
        return out, lse
    need = decode_workspace_bytes(g, B, N, step0, n_steps)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    st = _lib.lib().loopvq_decode_attn(
        ctypes.byref(g), _ptr(q), step0, n_steps, _ptr(k_idx), _ptr(v_idx), N_cap, _ptr(k_cb), _ptr(v_cb),
        _ptr(sink_k), _ptr(sink_v), n_s, _ptr(recent_k), _ptr(recent_v), n_r, R_cap, B, N, _ptr(seq_len),
        ctypes.byref(pt) if pt is not None else None,
        _ptr(rope), rope.shape[0], _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    check(st)
    return out, lse


def rope_table_f32(n_pos, D=128, theta=1.0e4, device="cuda", stream=None):
    """fp32 [n_pos][D/2][2]: (cos, sin) of angle p * theta^(-2f/D), computed in fp64."""
    t = torch.empty((n_pos, D // 2, 2), dtype=torch.float32, device=device)
    check(_lib.lib().loopvq_rope_table_f32(theta, D, n_pos, _ptr(t), _stream(stream)))
    return t


def _prefill_common(g, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, pt=None):
    _need(q, torch.float32, "q")
    _need(k_idx, torch.uint8, "k_idx")
    _need(v_idx, torch.uint8, "v_idx")
    _need(k_cb, torch.bfloat16, "k_cb")
    _need(v_cb, torch.bfloat16, "v_cb")
    _need(rope, torch.float32, "rope")
    for t, n in ((q, "q"), (k_idx, "k_idx"), (v_idx, "v_idx"), (k_cb, "k_cb"), (v_cb, "v_cb"), (rope, "rope")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    if q.dim() != 5:
        raise ValueError("q must be [B][Hq][n_steps][N][D]")
    B, _, n_steps, N, _ = q.shape
    n_blk, cpt = _dims(g)
    _shape(q, (B, g.n_q_heads, n_steps, N, g.D), "q")
    _shape(k_idx, (B, g.n_kv_heads, n_blk, None, cpt), "k_idx")
    _shape(v_idx, tuple(k_idx.shape), "v_idx")
    if k_idx.shape[3] < N:
        raise ValueError("k_idx holds %d tokens, q has %d positions" % (k_idx.shape[3], N))
    _shape(k_cb, (g.n_kv_heads, n_blk, g.K, g.G), "k_cb")
    _shape(v_cb, (g.n_kv_heads, n_blk, g.K, g.G), "v_cb")
    _shape(rope, (None, g.D // 2, 2), "rope")
    n_s = 0
    if (sink_k is None) != (sink_v is None):
        raise ValueError("sink_k and sink_v must both be given or both be None")
    if sink_k is not None:
        _need(sink_k, torch.bfloat16, "sink_k")
        _need(sink_v, torch.bfloat16, "sink_v")
        n_s = sink_k.shape[3]
        _shape(sink_k, (B, g.n_kv_heads, g.T, n_s, g.D), "sink_k")
        _shape(sink_v, (B, g.n_kv_heads, g.T, n_s, g.D), "sink_v")
        if not sink_k.is_contiguous() or not sink_v.is_contiguous():
            raise ValueError("sink_k and sink_v must be contiguous")
    _check_pt(g, pt, B, N)
    return n_s


def prefill_attn(g: Geom, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, step0=0, out=None, lse=None,
                 pt=None, stream=None):
    """Causal attention of the N positions after the sinks over the compressed cache.
    q fp32 [B][Hq][n_steps][N][D] (post-RoPE, query i at position n_s + i); k_idx/v_idx uint8
    [B][H][n_blk][N_cap][D/c]; k_cb/v_cb bf16 [H][n_blk][K][G]; sinks bf16 [B][H][T][n_s][D] or
    None; rope fp32 table from rope_table_f32(); pt the keys' pre-transform (pretransform()) or None.
    Returns (out fp32 like q, lse fp32 [B][Hq][n_steps][N])."""
    n_s = _prefill_common(g, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, pt)
    B, Hq, n_steps, N, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, n_steps, N), dtype=torch.float32, device=q.device)
    check(_lib.lib().loopvq_prefill_attn(
        ctypes.byref(g), _ptr(q), step0, n_steps, B, N, _ptr(k_idx), _ptr(v_idx), k_idx.shape[3], _ptr(k_cb),
        _ptr(v_cb), _ptr(sink_k), _ptr(sink_v), n_s, ctypes.byref(pt) if pt is not None else None, _ptr(rope),
        rope.shape[0], _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def prefill_attn_backward(g: Geom, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, out, lse, d_out,
                          step0=0, d_q=None, d_k_cb=None, d_v_cb=None, workspace=None, pt=None, stream=None):
    """Gradients of prefill_attn: returns (d_q fp32 like q, d_k_cb, d_v_cb fp32 [H][n_blk][K][G]).
    The codebook gradients are overwritten (sums over every q-head, step and token in the call)."""
    n_s = _prefill_common(g, q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, rope, pt)
    for t, n in ((out, "out"), (lse, "lse"), (d_out, "d_out")):
        _need(t, torch.float32, n)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    B, Hq, n_steps, N, D = q.shape
    _shape(out, tuple(q.shape), "out")
    _shape(d_out, tuple(q.shape), "d_out")
    _shape(lse, (B, Hq, n_steps, N), "lse")
    if d_q is None:
        d_q = torch.empty_like(q)
    if d_k_cb is None:
        d_k_cb = torch.empty(k_cb.shape, dtype=torch.float32, device=q.device)
    if d_v_cb is None:
        d_v_cb = torch.empty(v_cb.shape, dtype=torch.float32, device=q.device)
    need = ctypes.c_size_t(0)
    check(_lib.lib().loopvq_prefill_attn_backward_workspace(ctypes.byref(g), B, N, step0, n_steps,
                                                            ctypes.byref(need)))
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(max(need.value, 16), dtype=torch.uint8, device=q.device)
    check(_lib.lib().loopvq_prefill_attn_backward(
        ctypes.byref(g), _ptr(q), step0, n_steps, B, N, _ptr(k_idx), _ptr(v_idx), k_idx.shape[3], _ptr(k_cb),
        _ptr(v_cb), _ptr(sink_k), _ptr(sink_v), n_s, ctypes.byref(pt) if pt is not None else None, _ptr(rope),
        rope.shape[0], _ptr(out), _ptr(lse), _ptr(d_out), _ptr(d_q), _ptr(d_k_cb), _ptr(d_v_cb), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return d_q, d_k_cb, d_v_cb


def _precise_common(g, q, k, v, sink_k, sink_v, rope):
    _need(q, torch.float32, "q")
    _need(k, torch.bfloat16, "k")
    _need(v, torch.bfloat16, "v")
    _need(rope, torch.float32, "rope")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (rope, "rope")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    if q.dim() != 5:
        raise ValueError("q must be [B][Hq][n_steps][N][D]")
    B, _, n_steps, N, _ = q.shape
    _shape(q, (B, g.n_q_heads, n_steps, N, g.D), "q")
    _shape(k, (B, g.n_kv_heads, g.T, None, g.D), "k")
    _shape(v, tuple(k.shape), "v")
    if k.shape[3] < N:
        raise ValueError("the cache holds %d tokens, q has %d positions" % (k.shape[3], N))
    _shape(rope, (None, g.D // 2, 2), "rope")
    n_s = 0
    if (sink_k is None) != (sink_v is None):
        raise ValueError("sink_k and sink_v must both be given or both be None")
    if sink_k is not None:
        _need(sink_k, torch.bfloat16, "sink_k")
        _need(sink_v, torch.bfloat16, "sink_v")
        n_s = sink_k.shape[3]
        _shape(sink_k, (B, g.n_kv_heads, g.T, n_s, g.D), "sink_k")
        _shape(sink_v, (B, g.n_kv_heads, g.T, n_s, g.D), "sink_v")
        if not sink_k.is_contiguous() or not sink_v.is_contiguous():
            raise ValueError("sink_k and sink_v must be contiguous")
    return n_s


def precise_attn(g: Geom, q, k, v, sink_k, sink_v, rope, step0=0, out=None, lse=None, stream=None):
    """Causal attention of the N positions after the sinks over the precise
    cache k, v bf16 [B][H][T][N_x][D] (pre-RoPE keys).  q fp32
    [B][Hq][n_steps][N][D] (post-RoPE); rope fp32 from rope_table_f32().
    Returns (out fp32 like q, lse fp32 [B][Hq][n_steps][N])."""
    n_s = _precise_common(g, q, k, v, sink_k, sink_v, rope)
    B, Hq, n_steps, N, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, n_steps, N), dtype=torch.float32, device=q.device)
    check(_lib.lib().loopvq_precise_attn(
        ctypes.byref(g), _ptr(q), step0, n_steps, B, N, _ptr(k), _ptr(v), k.shape[3], _ptr(sink_k), _ptr(sink_v),
        n_s, _ptr(rope), rope.shape[0], _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def precise_attn_backward(g: Geom, q, k, v, sink_k, sink_v, rope, out, lse, d_out, d_k, d_v, step0=0, d_q=None,
                          workspace=None, stream=None):
    """Gradients of precise_attn: returns d_q (fp32 like q); the gradients of
    the served steps' cached keys (pre-RoPE) and values are ADDED into d_k,
    d_v fp32 [B][H][T][N_x][D]."""
    n_s = _precise_common(g, q, k, v, sink_k, sink_v, rope)
    for t, n in ((out, "out"), (lse, "lse"), (d_out, "d_out"), (d_k, "d_k"), (d_v, "d_v")):
        _need(t, torch.float32, n)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    B, Hq, n_steps, N, D = q.shape
    _shape(out, tuple(q.shape), "out")
    _shape(d_out, tuple(q.shape), "d_out")
    _shape(lse, (B, Hq, n_steps, N), "lse")
    _shape(d_k, tuple(k.shape), "d_k")
    _shape(d_v, tuple(k.shape), "d_v")
    if d_q is None:
        d_q = torch.empty_like(q)
    need = max(16, B * Hq * n_steps * N * 4)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    check(_lib.lib().loopvq_precise_attn_backward(
        ctypes.byref(g), _ptr(q), step0, n_steps, B, N, _ptr(k), _ptr(v), k.shape[3], _ptr(sink_k), _ptr(sink_v),
        n_s, _ptr(rope), rope.shape[0], _ptr(out), _ptr(lse), _ptr(d_out), _ptr(d_q), _ptr(d_k), _ptr(d_v),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return d_q


def fisher_weights(g: Geom, d_k, d_v, N=None, pt=None, omega_k=None, omega_v=None, stream=None):
    """Importance of every joint vector (sum of its squared gradient
    coordinates) from the cache gradients d_k, d_v fp32 [B][H][T][N_x][D].
    Returns (omega_k, omega_v) fp32 [B][H][n_blk][N][D/c], the weights of
    kmeans_accumulate."""
    _need(d_k, torch.float32, "d_k")
    _need(d_v, torch.float32, "d_v")
    if not d_k.is_contiguous() or not d_v.is_contiguous():
        raise ValueError("d_k and d_v must be contiguous")
    B = d_k.shape[0]
    _shape(d_k, (B, g.n_kv_heads, g.T, None, g.D), "d_k")
    _shape(d_v, tuple(d_k.shape), "d_v")
    N_x = d_k.shape[3]
    N = N_x if N is None else N
    n_blk, cpt = _dims(g)
    shp = (B, g.n_kv_heads, n_blk, N, cpt)
    if omega_k is None:
        omega_k = torch.empty(shp, dtype=torch.float32, device=d_k.device)
    if omega_v is None:
        omega_v = torch.empty(shp, dtype=torch.float32, device=d_k.device)
    for t, n in ((omega_k, "omega_k"), (omega_v, "omega_v")):
        _need(t, torch.float32, n)
        _shape(t, shp, n)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    _check_pt(g, pt, B, N)
    check(_lib.lib().loopvq_fisher_weights(ctypes.byref(g), _ptr(d_k), _ptr(d_v), B, N, N_x,
                                           ctypes.byref(pt) if pt is not None else None, _ptr(omega_k),
                                           _ptr(omega_v), _stream(stream)))
    return omega_k, omega_v
