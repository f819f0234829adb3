"""ctypes loader for libctxattn.so: argument types of every exported entry point.

The library is built in-tree by ``context_attention_lse_amd._build``. If it is
missing, loading fails loudly: there is no fallback implementation.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libctxattn.so")

CA_OK, CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_WORKSPACE, CA_ERR_HIP = range(7)
CA_BF16, CA_FP32 = 0, 1
CA_MASK_NONE, CA_MASK_CAUSAL_INCL, CA_MASK_CAUSAL_STRICT = 0, 1, 2
CA_PHASE_ACCUMULATE, CA_PHASE_INIT, CA_PHASE_FINAL = 0, 1, 2

STATUS_NAMES = {
    CA_OK: "CA_OK", CA_ERR_NULL: "CA_ERR_NULL", CA_ERR_SHAPE: "CA_ERR_SHAPE", CA_ERR_DTYPE: "CA_ERR_DTYPE",
    CA_ERR_UNSUPPORTED: "CA_ERR_UNSUPPORTED", CA_ERR_WORKSPACE: "CA_ERR_WORKSPACE", CA_ERR_HIP: "CA_ERR_HIP",
}

# Every symbol include/ctxattn.h declares.
EXPORTS = (
    "ring_attn_step", "ring_attn_step_fold", "ring_attn_step_hop", "ring_attn_step_fold_hop", "ring_attn_workspace_size", "key_sqnorm_max", "const_max_bound", "ring_attn_const_max_step", "ring_attn_const_max_step_hop", "lse_merge",
    "dcp_decode_partial", "dcp_decode_partial_active", "dcp_decode_workspace_size", "kv_chunk_copy", "ca_last_error",
    "ca_version", "segmented_attention_partial", "segmented_attention_workspace_size", "const_max_sink_prologue",
    "ring_attn_const_max_step_sinks", "sink_attention_partial", "sink_attention_workspace_size",
    "dcp_decode_partial_noalloc", "ring_attn_step_pair",
)


class ca_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("s", ctypes.c_int64), ("h", ctypes.c_int64)]


_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

SIGNATURES = {
    "ring_attn_step": [_vp, ca_strides, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _sz,
                       _vp],
    "ring_attn_step_fold": [_vp, ca_strides, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp,
                            _sz, _vp],
    "ring_attn_step_hop": [_vp, ca_strides, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp,
                           _sz, _vp, _vp, _vp, _vp, _sz, _vp],
    "ring_attn_step_fold_hop": [_vp, ca_strides, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp,
                                _vp, _sz, _vp, _vp, _vp, _vp, _sz, _vp],
    "ring_attn_step_pair": [_vp, ca_strides, _vp, _vp, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp,
                            _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "ring_attn_workspace_size": [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)],
    "key_sqnorm_max": [_vp, ca_strides, _i, _i, _i, _i, _i, _vp, _i, _vp],
    "const_max_bound": [_vp, ca_strides, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp],
    "ring_attn_const_max_step": [_vp, ca_strides, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i,
                                 _vp, _i, _vp, _vp, _sz, _vp],
    "ring_attn_const_max_step_hop": [_vp, ca_strides, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                     _i, _vp, _i, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _sz, _vp],
    "lse_merge": [_i, _vp, _vp, _i64, _i, _vp, _i, _vp, _vp],
    "dcp_decode_partial": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _vp],
    "dcp_decode_partial_noalloc": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp],
    "dcp_decode_partial_active": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                                  _vp, _vp, _sz, _vp],
    "dcp_decode_workspace_size": [_i, _i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)],
    "kv_chunk_copy": [_vp, _vp, _vp, _vp, _sz, _vp],
    "segmented_attention_partial": [_vp, ca_strides, _vp, _vp, ca_strides, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                    _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _vp],
    "segmented_attention_workspace_size": [_i, _i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)],
    "const_max_sink_prologue": [_vp, _i64, ca_strides, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _vp, _vp, _vp],
    "ring_attn_const_max_step_sinks": [_vp, ca_strides, _vp, _vp, ca_strides, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                       _i, _vp, _i, _vp, _vp, _vp, _i, _i64, _vp, _sz, _vp],
    "sink_attention_partial": [_vp, ca_strides, _vp, _vp, _i64, ca_strides, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i,
                               _vp, _vp, _vp, _sz, _vp],
    "sink_attention_workspace_size": [_i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)],
    "ca_last_error": [],
    "ca_version": [],
}

_LIB = None


class CtxAttnError(RuntimeError):
    def __init__(self, fn, status, message):
        super().__init__(f"{fn} failed with {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.fn = fn


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads (once) and returns the library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"libctxattn.so not found at {path}: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950). "
            "There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("ca_last_error", "ca_version") else ctypes.c_int
    _LIB = lib
    return lib


def call(name: str, *args) -> None:
    lib = load()
    st = getattr(lib, name)(*args)
    if st != CA_OK:
        msg = lib.ca_last_error().decode(errors="replace")
        raise CtxAttnError(name, st, msg)
