"""LoopVQ hot path on MI355X: loop-axis VQ encode and fused decode attention.

The compute lives in libloopvq.so (hand-written HIP for gfx950) behind a C ABI
(include/loopvq.h); this package only marshals torch tensors into it.
"""
from ._lib import LoopVQError, lib  # noqa: F401
from .api import (decode_attn, decode_attn_noalloc, decode_workspace_bytes, encode, fisher_weights,  # noqa: F401
                  geom, kmeans_accumulate, kmeans_finalize, precise_attn, precise_attn_backward, prefill_attn,
                  prefill_attn_backward, pretransform, rope_table, rope_table_f32, tasq_covariance,
                  tasq_pair_permutation)
