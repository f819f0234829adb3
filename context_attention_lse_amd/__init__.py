"""MI355X-native core of context-parallel attention with LSE merging.

One rank's share of ring attention (online-max or const-max steps over K/V chunks),
the LSE-corrected merge, and DCP decode over interleaved paged KV shards, computed by
hand-written HIP kernels for gfx950 in libctxattn.so (C ABI: include/ctxattn.h).
This package is the Python binding (argument marshalling) plus the host-side ring
and DCP drivers that order the library's calls.
"""

from .api import (  # noqa: F401
    CtxAttnError,
    const_max_acc_size,
    const_max_bound,
    const_max_sink_prologue,
    dcp_decode_partial,
    dcp_decode_partial_active,
    dcp_decode_partial_noalloc,
    dcp_decode_workspace_size,
    key_sqnorm_max,
    kv_chunk_copy,
    lse_merge,
    ring_attn_const_max_step,
    ring_attn_step,
    ring_attn_step_pair,
    ring_attn_workspace_size,
    segmented_attention_partial,
    segmented_attention_workspace_size,
    sink_attention_partial,
    sink_attention_workspace_size,
    step_workspace,
    version,
)
from . import dcp, ring, streams  # noqa: F401

__all__ = [
    "CtxAttnError", "const_max_acc_size", "const_max_bound", "dcp_decode_partial", "dcp_decode_partial_active", "dcp_decode_partial_noalloc",
    "dcp_decode_workspace_size",
    "key_sqnorm_max", "kv_chunk_copy", "lse_merge", "ring_attn_const_max_step", "ring_attn_step", "ring_attn_step_pair",
    "ring_attn_workspace_size",
    "segmented_attention_partial", "segmented_attention_workspace_size", "const_max_sink_prologue",
    "sink_attention_partial", "sink_attention_workspace_size", "step_workspace", "version",
    "dcp", "ring",
]
