"""ctypes loader for libloopvq.so (built in-tree by sub_bit_loop_amd/build.py).

Raises ImportError when the library is missing: there is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libloopvq.so")

OK, EINVAL, ENOTSUP, EHIP, EWORKSPACE = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 8 << 20     # LOOPVQ_NOALLOC_SCRATCH_BYTES
STATUS_NAME = {OK: "OK", EINVAL: "EINVAL", ENOTSUP: "ENOTSUP", EHIP: "EHIP", EWORKSPACE: "EWORKSPACE"}

# Names the C header declares; tests check that every one is exported.
EXPORTS = ("loopvq_encode", "loopvq_rope_table", "loopvq_decode_attn_workspace",
           "loopvq_decode_attn", "loopvq_decode_attn_noalloc", "loopvq_tasq_covariance", "loopvq_tasq_pair_permutation",
           "loopvq_kmeans_accumulate", "loopvq_kmeans_finalize", "loopvq_rope_table_f32",
           "loopvq_prefill_attn", "loopvq_prefill_attn_backward_workspace", "loopvq_prefill_attn_backward",
           "loopvq_precise_attn", "loopvq_precise_attn_backward", "loopvq_fisher_weights",
           "loopvq_last_error", "loopvq_abi_version")


class Geom(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("T", ctypes.c_int32), ("T_c", ctypes.c_int32),
                ("G", ctypes.c_int32), ("K", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("rope_theta", ctypes.c_float)]


class PreTransform(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("sigma", ctypes.c_void_p),
                ("N_cap", ctypes.c_int32)]


class LoopVQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS_NAME.get(status, status), msg))
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libloopvq.so is not built (run sub_bit_loop_amd/build.py); "
                          "the LoopVQ path has no fallback")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64P, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_size_t
    GP, PTP = ctypes.POINTER(Geom), ctypes.POINTER(PreTransform)
    L.loopvq_encode.argtypes = [GP, P, I64P, P, I32, I32, I32, P, I32, PTP, P]
    L.loopvq_encode.restype = ctypes.c_int
    L.loopvq_rope_table.argtypes = [ctypes.c_float, I32, I32, P, P]
    L.loopvq_rope_table.restype = ctypes.c_int
    L.loopvq_decode_attn_workspace.argtypes = [GP, I32, I32, I32, I32, ctypes.POINTER(SZ)]
    L.loopvq_decode_attn_workspace.restype = ctypes.c_int
    L.loopvq_decode_attn.argtypes = [GP, P, I32, I32, P, P, I32, P, P, P, P, I32, P, P, I32, I32,
                                     I32, I32, P, PTP, P, I32, P, P, P, SZ, P]
    L.loopvq_decode_attn.restype = ctypes.c_int
    L.loopvq_decode_attn_noalloc.argtypes = [GP, P, I32, I32, P, P, I32, P, P, P, P, I32, P, P, I32, I32,
                                             I32, I32, P, PTP, P, I32, P, P, P]
    L.loopvq_decode_attn_noalloc.restype = ctypes.c_int
    L.loopvq_tasq_covariance.argtypes = [GP, P, I64P, I32, I32, P, P, I32, P, P, P]
    L.loopvq_tasq_covariance.restype = ctypes.c_int
    L.loopvq_tasq_pair_permutation.argtypes = [P, I32, I32, I32, P]
    L.loopvq_tasq_pair_permutation.restype = ctypes.c_int
    L.loopvq_kmeans_accumulate.argtypes = [GP, P, I64P, I32, I32, P, I32, P, PTP, P, P, P]
    L.loopvq_kmeans_accumulate.restype = ctypes.c_int
    L.loopvq_kmeans_finalize.argtypes = [GP, P, P, P, P]
    L.loopvq_kmeans_finalize.restype = ctypes.c_int
    L.loopvq_rope_table_f32.argtypes = [ctypes.c_float, I32, I32, P, P]
    L.loopvq_rope_table_f32.restype = ctypes.c_int
    L.loopvq_prefill_attn.argtypes = [GP, P, I32, I32, I32, I32, P, P, I32, P, P, P, P, I32, PTP, P, I32, P, P, P]
    L.loopvq_prefill_attn.restype = ctypes.c_int
    L.loopvq_prefill_attn_backward_workspace.argtypes = [GP, I32, I32, I32, I32, ctypes.POINTER(SZ)]
    L.loopvq_prefill_attn_backward_workspace.restype = ctypes.c_int
    L.loopvq_prefill_attn_backward.argtypes = [GP, P, I32, I32, I32, I32, P, P, I32, P, P, P, P, I32, PTP, P,
                                               I32, P, P, P, P, P, P, P, SZ, P]
    L.loopvq_prefill_attn_backward.restype = ctypes.c_int
    L.loopvq_precise_attn.argtypes = [GP, P, I32, I32, I32, I32, P, P, I32, P, P, I32, P, I32, P, P, P]
    L.loopvq_precise_attn.restype = ctypes.c_int
    L.loopvq_precise_attn_backward.argtypes = [GP, P, I32, I32, I32, I32, P, P, I32, P, P, I32, P, I32, P, P, P,
                                               P, P, P, P, SZ, P]
    L.loopvq_precise_attn_backward.restype = ctypes.c_int
    L.loopvq_fisher_weights.argtypes = [GP, P, P, I32, I32, I32, PTP, P, P, P]
    L.loopvq_fisher_weights.restype = ctypes.c_int
    L.loopvq_last_error.argtypes = []
    L.loopvq_last_error.restype = ctypes.c_char_p
    L.loopvq_abi_version.argtypes = []
    L.loopvq_abi_version.restype = ctypes.c_int32
    _lib = L
    return L


def check(status):
    if status != OK:
        msg = lib().loopvq_last_error().decode(errors="replace")
        raise LoopVQError(status, msg)
