"""C ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments on the host before any
HIP call with the documented status codes."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from sub_bit_loop_amd import _lib as L
    return L, L.lib()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "loopvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(loopvq_[a-z0-9_]+)\s*\(", src)))


def test_exports_match_header():
    L, lib = _lib()
    names = _header_functions()
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.loopvq_abi_version() == 4


def _geom(L, **kw):
    d = dict(D=128, T=4, T_c=4, G=16, K=256, n_kv_heads=2, n_q_heads=4, rope_theta=1e4)
    d.update(kw)
    return L.Geom(**d)


BAD_GEOMS = [
    (dict(T_c=3), -1), (dict(T=6, T_c=4), -1), (dict(G=18), -1), (dict(K=1), -1), (dict(K=257), -1),
    (dict(n_q_heads=3), -1), (dict(rope_theta=0.0), -1), (dict(D=127), -1), (dict(D=64), -2),
    (dict(G=8, T_c=4), -2), (dict(T=32, T_c=16, G=16), -2), (dict(G=24, T_c=4), -1), (dict(G=64, T_c=4), -2),
]


@pytest.mark.parametrize("over,code", BAD_GEOMS)
def test_encode_rejects_geometry(over, code):
    L, lib = _lib()
    g = _geom(L, **over)
    strides = (ctypes.c_int64 * 4)(512, 512, 128, 128)
    st = lib.loopvq_encode(ctypes.byref(g), ctypes.c_void_p(16), strides, ctypes.c_void_p(16), 1, 4, 0,
                           ctypes.c_void_p(16), 4, None, None)
    assert st == code
    assert len(lib.loopvq_last_error()) > 0


def test_encode_argument_errors():
    L, lib = _lib()
    g = _geom(L)
    P = ctypes.c_void_p
    good = (ctypes.c_int64 * 4)(4096, 2048, 512, 128)
    # N = 0 is a no-op even with NULL tensors
    assert lib.loopvq_encode(ctypes.byref(g), None, None, None, 1, 0, 0, None, 0, None, None) == 0
    cases = [
        (P(0), good, P(16), 1, 4, 0, P(16), 4),                       # NULL x
        (P(16), good, P(16), -1, 4, 0, P(16), 4),                     # negative B
        (P(16), good, P(16), 1, 4, 1, P(16), 4),                      # tok0 + N > N_cap
        (P(16), (ctypes.c_int64 * 4)(4096, 2048, 512, 0), P(16), 1, 4, 0, P(16), 4),  # zero stride
        (P(16), (ctypes.c_int64 * 4)(4096, 2048, 512, 129), P(16), 1, 4, 0, P(16), 4),  # odd stride
        (P(8), good, P(16), 1, 4, 0, P(16), 4),                       # misaligned x
    ]
    for x, st, cb, B, N, tok0, idx, cap in cases:
        assert lib.loopvq_encode(ctypes.byref(g), x, st, cb, B, N, tok0, idx, cap, None, None) == -1
    pt = L.PreTransform(16, 0, 16, 4)                                  # NULL perm
    assert lib.loopvq_encode(ctypes.byref(g), P(16), good, P(16), 1, 4, 0, P(16), 4, ctypes.byref(pt), None) == -1
    pt = L.PreTransform(16, 16, 16, 2)                                 # sigma capacity too small
    assert lib.loopvq_encode(ctypes.byref(g), P(16), good, P(16), 1, 4, 0, P(16), 4, ctypes.byref(pt), None) == -1


def test_rope_table_argument_errors():
    L, lib = _lib()
    P = ctypes.c_void_p
    assert lib.loopvq_rope_table(1e4, 128, 10, P(0), None) == -1
    assert lib.loopvq_rope_table(1e4, 127, 10, P(16), None) == -1
    assert lib.loopvq_rope_table(1e4, 132, 10, P(16), None) == -1
    assert lib.loopvq_rope_table(1e4, 128, 0, P(16), None) == -1
    assert lib.loopvq_rope_table(-1.0, 128, 10, P(16), None) == -1


def test_decode_workspace_and_errors():
    L, lib = _lib()
    g = _geom(L)
    sz = ctypes.c_size_t(0)
    assert lib.loopvq_decode_attn_workspace(ctypes.byref(g), 2, 1000, 0, 4, ctypes.byref(sz)) == 0
    # 2 x 4 q-heads x 4 steps rows, four context splits of D + 1 floats each
    assert sz.value == 2 * 4 * 4 * 4 * 129 * 4
    assert lib.loopvq_decode_attn_workspace(ctypes.byref(g), 2, 1000, 3, 2, ctypes.byref(sz)) == -1
    assert lib.loopvq_decode_attn_workspace(ctypes.byref(g), 2, 1000, 0, 0, ctypes.byref(sz)) == -1
    P = ctypes.c_void_p
    need = ctypes.c_size_t(0)
    lib.loopvq_decode_attn_workspace(ctypes.byref(g), 2, 100, 0, 4, ctypes.byref(need))

    def call(**kw):
        a = dict(q=P(16), step0=0, n_steps=4, k_idx=P(16), v_idx=P(16), N_cap=100, k_cb=P(16), v_cb=P(16),
                 sink_k=P(16), sink_v=P(16), n_s=4, rk=P(16), rv=P(16), n_r=8, R_cap=8, B=2, N=100,
                 seq_len=None, pt=None, rope=P(16), n_pos=112, out=P(16), lse=P(16), ws=P(16),
                 ws_bytes=need.value)
        a.update(kw)
        return lib.loopvq_decode_attn(ctypes.byref(g), a["q"], a["step0"], a["n_steps"], a["k_idx"], a["v_idx"],
                                      a["N_cap"], a["k_cb"], a["v_cb"], a["sink_k"], a["sink_v"], a["n_s"],
                                      a["rk"], a["rv"], a["n_r"], a["R_cap"], a["B"], a["N"], a["seq_len"],
                                      a["pt"], a["rope"], a["n_pos"], a["out"], a["lse"], a["ws"],
                                      a["ws_bytes"], None)
    assert call(q=P(0)) == -1
    assert call(N=101) == -1                  # N > N_cap
    assert call(n_pos=111) == -1              # table too short for sinks + N + recent
    assert call(n_r=9) == -1                  # n_r > R_cap
    assert call(rk=P(0)) == -1                # recent window missing with n_r > 0
    assert call(sink_k=P(0)) == -1            # sinks missing with n_s > 0
    assert call(k_cb=P(8)) == -1              # misaligned codebook
    assert call(step0=2, n_steps=3) == -1     # step range outside [0, T)
    assert call(n_s=-1) == -1
    assert call(ws_bytes=need.value - 1) == -4
    assert call(ws=P(0)) == -4
    assert call(B=0) == 0                     # nothing to do
    # pre-transformed keys: the kernel's index-row, sigma and table offsets are
    # 32-bit, so a capacity of 2^26 tokens of 32-byte rows (2^31 bytes) is refused
    big = 1 << 26
    pt = L.PreTransform(16, 16, 16, big)
    wide = ctypes.c_size_t(0)
    assert lib.loopvq_decode_attn_workspace(ctypes.byref(g), 2, 100, 0, 4, ctypes.byref(wide)) == 0
    assert call(N_cap=big, pt=ctypes.byref(pt), ws_bytes=wide.value) == -2
    assert "32-bit" in lib.loopvq_last_error().decode()
    assert call(N_cap=big - 1, pt=ctypes.byref(pt), ws_bytes=wide.value, q=P(0)) == -1   # plain argument errors first


def test_kmeans_entry_points_reject_bad_arguments():
    import sub_bit_loop_amd as lv
    _, lib = _lib()
    g = lv.geom(128, 4, 4, 16, 256, 1, 1)
    P = ctypes.c_void_p
    st = (ctypes.c_int64 * 4)(4 * 8 * 128, 4 * 8 * 128, 8 * 128, 128)
    P16 = P(16)
    # N > N_cap, negative B, NULL outputs: all refused on the host
    assert lib.loopvq_kmeans_accumulate(ctypes.byref(g), P16, st, 1, 9, P16, 8, None, None, P16, P16, None) == -1
    assert lib.loopvq_kmeans_accumulate(ctypes.byref(g), P16, st, -1, 8, P16, 8, None, None, P16, P16, None) == -1
    assert lib.loopvq_kmeans_accumulate(ctypes.byref(g), P16, st, 1, 8, P16, 8, None, None, None, P16, None) == -1
    # nothing to do
    assert lib.loopvq_kmeans_accumulate(ctypes.byref(g), None, None, 1, 0, None, 8, None, None, None, None, None) == 0
    assert lib.loopvq_kmeans_finalize(ctypes.byref(g), None, P16, P16, None) == -1
    bad = lv.geom(128, 4, 4, 24, 256, 1, 1)
    assert lib.loopvq_kmeans_finalize(ctypes.byref(bad), P16, P16, P16, None) != 0


def test_prefill_entry_points_reject_bad_arguments():
    import sub_bit_loop_amd as lv
    _, lib = _lib()
    g = lv.geom(128, 4, 4, 16, 256, 2, 4)
    P = ctypes.c_void_p
    A = P(256)                 # stands in for an aligned device pointer; never dereferenced
    U = P(258)                 # misaligned
    # prefill_attn(g, q, step0, n_steps, B, N, kidx, vidx, N_cap, kcb, vcb, sk, sv, n_s, pt, rope, n_pos, out,
    #              lse, s)
    ok = [A, 0, 4, 1, 8, A, A, 8, A, A, A, A, 4, None, A, 12, A, A, None]

    def fwd(**ch):
        args = list(ok)
        names = ["q", "step0", "n_steps", "B", "N", "kidx", "vidx", "N_cap", "kcb", "vcb", "sk", "sv", "n_s",
                 "pt", "rope", "n_pos", "out", "lse", "s"]
        for k, v in ch.items():
            args[names.index(k)] = v
        return lib.loopvq_prefill_attn(ctypes.byref(g), *args)
    assert fwd(q=None) == -1
    assert fwd(N=9) == -1                  # N > N_cap
    assert fwd(n_pos=11) == -1             # rope table shorter than n_s + N
    assert fwd(step0=1) == -1              # step range beyond T
    assert fwd(sk=None) == -1              # n_s > 0 without sinks
    assert fwd(q=U) == -1                  # misaligned
    assert fwd(lse=None) == -1
    assert fwd(N=0) == 0                   # nothing to attend: no launch
    assert fwd(n_s=-1) == -1
    # a pre-transform with a NULL member is refused
    bad_pt = lv.pretransform.__globals__["PreTransform"](None, None, None, 8)
    assert fwd(pt=ctypes.byref(bad_pt)) == -1
    bad = lv.geom(128, 4, 4, 24, 256, 2, 4)
    assert lib.loopvq_prefill_attn(ctypes.byref(bad), *ok) != 0
    size = ctypes.c_size_t(0)
    assert lib.loopvq_prefill_attn_backward_workspace(ctypes.byref(g), 2, 8, 0, 4, ctypes.byref(size)) == 0
    assert size.value == 2 * 4 * 4 * 8 * 4
    # backward: short workspace and NULL gradients are refused before any launch
    bargs = [A, 0, 4, 1, 8, A, A, 8, A, A, A, A, 4, None, A, 12, A, A, A, A, A, A, A, 16, None]
    assert lib.loopvq_prefill_attn_backward(ctypes.byref(g), *bargs) == -4
    bargs[23] = 1 * 4 * 4 * 8 * 4
    bargs[20] = None
    assert lib.loopvq_prefill_attn_backward(ctypes.byref(g), *bargs) == -1
    assert lib.loopvq_rope_table_f32(1e4, 7, 4, A, None) == -1
    assert lib.loopvq_rope_table_f32(1e4, 128, 0, A, None) == -1
