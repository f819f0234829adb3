"""Python binding of libctxattn: the C entry points under the same names.

Argument marshalling only. Each function checks devices and dtypes, allocates the
outputs it is not given (with torch, the caller-side allocator), and passes raw
pointers, sizes and the current HIP stream to the library. Every computation runs
in the library's HIP kernels; there is no other implementation to fall back to.

Tensors follow the library's layouts: attention inputs are [B, S, H, D] (any
strides with D contiguous), outputs [B, H, S, D] fp32 and LSE [B, H, S] fp32.
"""

import ctypes

import torch

from . import _lib
from ._lib import (CA_BF16, CA_FP32, CA_MASK_CAUSAL_INCL, CA_MASK_CAUSAL_STRICT, CA_MASK_NONE,  # noqa: F401
                   CA_PHASE_ACCUMULATE, CA_PHASE_FINAL, CA_PHASE_INIT, CtxAttnError)

MASKS = {"none": CA_MASK_NONE, "causal_incl": CA_MASK_CAUSAL_INCL, "causal_strict": CA_MASK_CAUSAL_STRICT}
_DT = {torch.bfloat16: CA_BF16, torch.float32: CA_FP32}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")
    return _DT[t.dtype]


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t: torch.Tensor) -> _lib.ca_strides:
    if t.dim() != 4:
        raise ValueError(f"expected a [B, S, H, D] tensor, got shape {tuple(t.shape)}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the head dimension D must be contiguous")
    return _lib.ca_strides(t.stride(0), t.stride(1), t.stride(2))


def _check_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _scale(scale):
    return 0.0 if scale is None else float(scale)


def ring_attn_workspace_size(dtype, B, H, Sq, Sk, D, mask="none") -> int:
    """Bytes of key-split workspace a step of these sizes needs on the current device (0: none)."""
    n = ctypes.c_size_t(0)
    code = _DT[dtype] if not isinstance(dtype, int) else dtype
    _lib.call("ring_attn_workspace_size", code, B, H, Sq, Sk, D, MASKS[mask] if isinstance(mask, str) else int(mask),
              ctypes.byref(n))
    return int(n.value)


def step_workspace(q, k, mask="none"):
    """A zeroed key-split workspace for steps of q's and k's shapes, or None if they never split.
    Reusable by any number of such steps in stream order; concurrent steps need their own."""
    B, Sq, H, D = q.shape
    n = ring_attn_workspace_size(q.dtype, B, H, Sq, k.shape[1], D, mask)
    return torch.zeros(n, dtype=torch.uint8, device=q.device) if n else None


def _ws(workspace):
    if workspace is None:
        return None, 0
    if not (workspace.is_contiguous() and workspace.dtype == torch.uint8):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    return _ptr(workspace), workspace.numel()


def _hop_bytes(hop):
    """Checks a hop (dst_k, dst_v, src_k, src_v) and returns its size in bytes."""
    _check_cuda(*hop)
    nbytes = hop[2].numel() * hop[2].element_size()
    for t in hop:
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous():
            raise ValueError("hop buffers must be contiguous and of one size")
    return nbytes


def ring_attn_step(q, k, v, scale=None, mask="none", out=None, lse=None, workspace=None, stream=None,
                   fold=False, hop=None):
    """Online-max attention of q [B, Sq, H, D] against one K/V chunk [B, Sk, H, D].
    Returns (o [B, H, Sq, D] fp32, lse [B, H, Sq] fp32). With ``workspace`` (from
    step_workspace) the key range is split over a grid that fills the device. With
    ``fold``, ``out`` and ``lse`` (required) hold a prior partial of the same rows and
    receive its LSE merge with this chunk's partial (ring_attn_step_fold). ``hop`` =
    (dst_k, dst_v, src_k, src_v), contiguous buffers of one size: the ring's next K/V hop,
    copied by the same call (ring_attn_step_hop, or ring_attn_step_fold_hop with ``fold``)."""
    _check_cuda(q, k, v, out, lse, workspace)
    if hop is not None:
        nbytes = _hop_bytes(hop)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    if q.dtype != k.dtype or k.dtype != v.dtype:
        raise TypeError("q, k and v must share a dtype")
    if fold:
        if out is None or lse is None:
            raise ValueError("fold needs the prior partial in out and lse")
        if out.shape != (B, H, Sq, D) or lse.shape != (B, H, Sq) or out.dtype != torch.float32 \
                or lse.dtype != torch.float32 or not (out.is_contiguous() and lse.is_contiguous()):
            raise ValueError("fold: out [B, H, Sq, D] and lse [B, H, Sq] must be contiguous fp32")
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _strides(q), _ptr(k), _ptr(v), _strides(k), _dtype_code(q), B, H, Sq, Sk, D, _scale(scale),
            MASKS[mask] if isinstance(mask, str) else int(mask), _ptr(out), _ptr(lse), *_ws(workspace))
    if hop is not None:
        _lib.call("ring_attn_step_fold_hop" if fold else "ring_attn_step_hop", *args, *(_ptr(t) for t in hop), nbytes,
                  _stream(stream))
    else:
        _lib.call("ring_attn_step_fold" if fold else "ring_attn_step", *args, _stream(stream))
    return out, lse


def ring_attn_step_pair(q, k1, v1, k2, v2, scale=None, out=None, lse=None, workspace=None, stream=None, fold=False,
                        hops=()):
    """Two consecutive ring steps in one launch: online-max attention of q [B, Sq, H, D] against
    the keys of chunk 1 and then of chunk 2 ([B, Sk1, H, D] and [B, Sk2, H, D], one set of
    strides, Sk1 a multiple of 32; no mask), i.e. the LSE merge of the two steps' partials.
    ``fold``, ``out``, ``lse``, ``workspace`` as for ring_attn_step. ``hops``: up to two ring
    hops (dst_k, dst_v, src_k, src_v) of one size, carried by the same launch."""
    _check_cuda(q, k1, v1, k2, v2, out, lse, workspace)
    hops = list(hops)
    if len(hops) > 2:
        raise ValueError("at most two hops")
    nbytes = 0
    for h in hops:
        n = _hop_bytes(h)
        if nbytes and n != nbytes:
            raise ValueError("the two hops must have one size")
        nbytes = n
    B, Sq, H, D = q.shape
    for k, v in ((k1, v1), (k2, v2)):
        if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
            raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
        if k.stride() != v.stride():
            raise ValueError("k and v must share strides")
    if k1.shape[1] and k2.shape[1] and k1.stride() != k2.stride():
        raise ValueError("both chunks must share strides")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise TypeError("q, k and v must share a dtype")
    if fold:
        if out is None or lse is None:
            raise ValueError("fold needs the prior partial in out and lse")
        if out.shape != (B, H, Sq, D) or lse.shape != (B, H, Sq) or out.dtype != torch.float32 \
                or lse.dtype != torch.float32 or not (out.is_contiguous() and lse.is_contiguous()):
            raise ValueError("fold: out [B, H, Sq, D] and lse [B, H, Sq] must be contiguous fp32")
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    hp = [_ptr(t) for h in hops for t in h] + [None] * (8 - 4 * len(hops))
    _lib.call("ring_attn_step_pair", _ptr(q), _strides(q), _ptr(k1), _ptr(v1), _ptr(k2), _ptr(v2),
              _strides(k1 if k1.shape[1] else k2),
              _dtype_code(q), B, H, Sq, k1.shape[1], k2.shape[1], D, _scale(scale), int(bool(fold)), _ptr(out),
              _ptr(lse), *_ws(workspace), *hp, nbytes, _stream(stream))
    return out, lse


def key_sqnorm_max(k, kmax_sq=None, accumulate=False, stream=None):
    """Per (b, h) max of |k_j|^2 over the chunk, optionally max-folded into kmax_sq [B, H]."""
    _check_cuda(k, kmax_sq)
    B, S, H, D = k.shape
    if kmax_sq is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing kmax_sq")
        kmax_sq = torch.empty((B, H), dtype=torch.float32, device=k.device)
    _lib.call("key_sqnorm_max", _ptr(k), _strides(k), _dtype_code(k), B, S, H, D, _ptr(kmax_sq),
              int(bool(accumulate)), _stream(stream))
    return kmax_sq


def const_max_bound(q, kmax_sq, scale=None, out=None, stream=None):
    """Per-row bound c [B, H, Sq] = scale * |q_i| * sqrt(kmax_sq[b, h])."""
    _check_cuda(q, kmax_sq, out)
    B, Sq, H, D = q.shape
    if out is None:
        out = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _lib.call("const_max_bound", _ptr(q), _strides(q), _dtype_code(q), B, Sq, H, D, _scale(scale),
              _ptr(kmax_sq), _ptr(out), _stream(stream))
    return out


def const_max_sink_prologue(k_pool, theta, sink_cap=32, out=None, stream=None):
    """Sink-robust bound prologue over a chunk pool [cp, B, S_local, H, D] (any strides with D
    contiguous). Returns dict(kmax_sq, kmax_sq_robust, knorm_sum [B, H] fp32,
    sink_idx [B, H, sink_cap] int32, sink_cnt [B, H] int32); ``out`` reuses such a dict."""
    _check_cuda(k_pool)
    cp, B, S, H, D = k_pool.shape
    dev = k_pool.device
    if out is None:
        out = {"kmax_sq": torch.empty((B, H), dtype=torch.float32, device=dev),
               "kmax_sq_robust": torch.empty((B, H), dtype=torch.float32, device=dev),
               "knorm_sum": torch.empty((B, H), dtype=torch.float32, device=dev),
               "sink_idx": torch.zeros((B, H, sink_cap), dtype=torch.int32, device=dev),
               "sink_cnt": torch.empty((B, H), dtype=torch.int32, device=dev)}
    st = k_pool.stride()
    _lib.call("const_max_sink_prologue", _ptr(k_pool), st[0], _lib.ca_strides(st[1], st[2], st[3]),
              _dtype_code(k_pool), cp, B, S, H, D, float(theta), int(sink_cap), _ptr(out["kmax_sq"]),
              _ptr(out["kmax_sq_robust"]), _ptr(out["knorm_sum"]), _ptr(out["sink_idx"]), _ptr(out["sink_cnt"]),
              _stream(stream))
    return out


def sink_attention_workspace_size(B, H, D, sink_cap) -> int:
    n = ctypes.c_size_t(0)
    _lib.call("sink_attention_workspace_size", B, H, D, int(sink_cap), ctypes.byref(n))
    return int(n.value)


def sink_attention_partial(q, k_pool, v_pool, sinks, scale=None, out=None, lse=None, workspace=None, stream=None):
    """Exact attention of q [B, Sq, H, D] against the listed sink keys of the pool alone.
    ``sinks``: the dict from const_max_sink_prologue. Returns (o [B, H, Sq, D], lse [B, H, Sq])."""
    _check_cuda(q, k_pool, v_pool, out, lse, workspace)
    cp, B, S, H, D = k_pool.shape
    Sq = q.shape[1]
    if k_pool.stride() != v_pool.stride() or k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must share shape and strides")
    cap = sinks["sink_idx"].shape[2]
    if workspace is None:
        workspace = torch.empty(max(16, sink_attention_workspace_size(B, H, D, cap)), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    st = k_pool.stride()
    _lib.call("sink_attention_partial", _ptr(q), _strides(q), _ptr(k_pool), _ptr(v_pool), st[0],
              _lib.ca_strides(st[1], st[2], st[3]), cp, B, H, Sq, S, D, _scale(scale), _ptr(sinks["sink_idx"]),
              _ptr(sinks["sink_cnt"]), cap, _ptr(out), _ptr(lse), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream))
    return out, lse


def const_max_acc_size(B, H, Sq, D) -> int:
    """Floats of the const-max accumulator: [B, H, Sq, D] output then [B, H, Sq] row sums."""
    return B * H * Sq * (D + 1)


def ring_attn_const_max_step(q, k, v, c, acc, phase, out=None, lse=None, out_dtype=torch.float32,
                             scale=None, workspace=None, stream=None, sinks=None, key_offset=0, hop=None):
    """One const-max ring step. acc: fp32 tensor of const_max_acc_size floats (None allowed
    when phase == INIT|FINAL). On the FINAL phase returns (o [B, H, Sq, D], lse [B, H, Sq]).
    ``workspace`` as for ring_attn_step. ``sinks`` (the dict from const_max_sink_prologue)
    leaves the listed keys out; ``key_offset`` is this chunk's first key index. ``hop`` as for
    ring_attn_step (ring_attn_const_max_step_hop; not with ``sinks``)."""
    _check_cuda(q, k, v, c, acc, out, lse, workspace)
    if hop is not None:
        if sinks is not None:
            raise ValueError("hop and sinks do not combine")
        nbytes = _hop_bytes(hop)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    if acc is not None and acc.numel() < const_max_acc_size(B, H, Sq, D):
        raise ValueError("acc is too small")
    final = bool(phase & CA_PHASE_FINAL)
    if final:
        if out is None:
            out = torch.empty((B, H, Sq, D), dtype=out_dtype, device=q.device)
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    o_args = (_ptr(out) if final else None, _DT.get(out.dtype, CA_FP32) if final else CA_FP32,
              _ptr(lse) if final else None)
    if hop is not None:
        _lib.call("ring_attn_const_max_step_hop", _ptr(q), _strides(q), _ptr(k), _ptr(v), _strides(k),
                  _dtype_code(q), B, H, Sq, Sk, D, _scale(scale), _ptr(c), _ptr(acc), int(phase), *o_args,
                  *_ws(workspace), *(_ptr(t) for t in hop), nbytes, _stream(stream))
    elif sinks is None:
        _lib.call("ring_attn_const_max_step", _ptr(q), _strides(q), _ptr(k), _ptr(v), _strides(k), _dtype_code(q),
                  B, H, Sq, Sk, D, _scale(scale), _ptr(c), _ptr(acc), int(phase), *o_args, *_ws(workspace),
                  _stream(stream))
    else:
        _lib.call("ring_attn_const_max_step_sinks", _ptr(q), _strides(q), _ptr(k), _ptr(v), _strides(k),
                  _dtype_code(q), B, H, Sq, Sk, D, _scale(scale), _ptr(c), _ptr(acc), int(phase), *o_args,
                  _ptr(sinks["sink_idx"]), _ptr(sinks["sink_cnt"]), sinks["sink_idx"].shape[2], int(key_offset),
                  *_ws(workspace), _stream(stream))
    return (out, lse) if final else None


def lse_merge(o_parts, lse_parts, out=None, lse_out=None, out_dtype=torch.float32, stream=None):
    """Merge n partials: o_parts [n, ..., D] fp32, lse_parts [n, ...] fp32 (contiguous).
    Returns (o [..., D], lse [...])."""
    _check_cuda(o_parts, lse_parts, out, lse_out)
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    n, D = o_parts.shape[0], o_parts.shape[-1]
    lead = tuple(o_parts.shape[1:-1])
    if tuple(lse_parts.shape) != (n,) + lead:
        raise ValueError(f"lse_parts shape {tuple(lse_parts.shape)} does not match {(n,) + lead}")
    rows = 1
    for x in lead:
        rows *= x
    if out is None:
        out = torch.empty(lead + (D,), dtype=out_dtype, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty(lead, dtype=torch.float32, device=o_parts.device)
    _lib.call("lse_merge", n, _ptr(o_parts), _ptr(lse_parts), rows, D, _ptr(out), _DT[out.dtype],
              _ptr(lse_out), _stream(stream))
    return out, lse_out


def dcp_decode_workspace_size(B, Hq, D, block_size, max_blocks) -> int:
    n = ctypes.c_size_t(0)
    _lib.call("dcp_decode_workspace_size", B, Hq, D, block_size, max_blocks, ctypes.byref(n))
    return int(n.value)


def dcp_decode_partial(q, k_pool, v_pool, block_table, local_lens, scale=None, out=None, lse=None,
                       workspace=None, stream=None):
    """One DCP shard's decode partial. q [B, Hq, D] bf16; k_pool [NB, Hkv, 16, D];
    v_pool [NB, Hkv, D, 16]; block_table [B, max_blocks] int32; local_lens [B] int32.
    Returns (o [B, Hq, D] fp32, lse [B, Hq] fp32)."""
    _check_cuda(q, k_pool, v_pool, block_table, local_lens, out, lse, workspace)
    B, Hq, D = q.shape
    NB, Hkv, bs, _ = k_pool.shape
    if tuple(v_pool.shape) != (NB, Hkv, D, bs):
        raise ValueError(f"v_pool must be [NB, Hkv, D, block_size], got {tuple(v_pool.shape)}")
    for t in (q, k_pool, v_pool, block_table, local_lens):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if block_table.dtype != torch.int32 or local_lens.dtype != torch.int32:
        raise TypeError("block_table and local_lens must be int32")
    if q.dtype != torch.bfloat16 or k_pool.dtype != torch.bfloat16 or v_pool.dtype != torch.bfloat16:
        raise TypeError("decode q and pools must be bfloat16")
    max_blocks = block_table.shape[1]
    need = dcp_decode_workspace_size(B, Hq, D, bs, max_blocks)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _lib.call("dcp_decode_partial", _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(local_lens),
              B, Hq, Hkv, D, bs, max_blocks, NB, _scale(scale), _ptr(out), _ptr(lse), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream))
    return out, lse


def dcp_decode_partial_noalloc(q, k_pool, v_pool, block_table, local_lens, scale=None, out=None, lse=None,
                               stream=None):
    """dcp_decode_partial without a workspace: the library's fixed per-GPU scratch holds the
    split partials, and the C call allocates nothing (the outputs are allocated here only if
    not given). Calls that may overlap in time on one GPU race on that scratch."""
    _check_cuda(q, k_pool, v_pool, block_table, local_lens, out, lse)
    B, Hq, D = q.shape
    NB, Hkv, bs, _ = k_pool.shape
    if tuple(v_pool.shape) != (NB, Hkv, D, bs):
        raise ValueError(f"v_pool must be [NB, Hkv, D, block_size], got {tuple(v_pool.shape)}")
    for t in (q, k_pool, v_pool, block_table, local_lens):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if block_table.dtype != torch.int32 or local_lens.dtype != torch.int32:
        raise TypeError("block_table and local_lens must be int32")
    if q.dtype != torch.bfloat16 or k_pool.dtype != torch.bfloat16 or v_pool.dtype != torch.bfloat16:
        raise TypeError("decode q and pools must be bfloat16")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _lib.call("dcp_decode_partial_noalloc", _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(local_lens),
              B, Hq, Hkv, D, bs, block_table.shape[1], NB, _scale(scale), _ptr(out), _ptr(lse), _stream(stream))
    return out, lse


def dcp_decode_partial_active(q, k_pool, v_pool, block_table, prior_lens, k_cur, v_cur, rank, world,
                              interleave=16, scale=None, out=None, lse=None, workspace=None, stream=None):
    """One DCP shard's decode step with the current token gated to its owner. q [B, Hq, D]
    bf16; pools and block_table as dcp_decode_partial (this shard's prior tokens);
    prior_lens [B] int32 (global prior count N); k_cur, v_cur [B, Hkv, D] bf16.
    Returns (o [B, Hq, D] fp32, lse [B, Hq] fp32)."""
    _check_cuda(q, k_pool, v_pool, block_table, prior_lens, k_cur, v_cur, out, lse, workspace)
    B, Hq, D = q.shape
    NB, Hkv, bs, _ = k_pool.shape
    if tuple(v_pool.shape) != (NB, Hkv, D, bs):
        raise ValueError(f"v_pool must be [NB, Hkv, D, block_size], got {tuple(v_pool.shape)}")
    if tuple(k_cur.shape) != (B, Hkv, D) or tuple(v_cur.shape) != (B, Hkv, D):
        raise ValueError(f"k_cur and v_cur must be [B, Hkv, D] = {(B, Hkv, D)}")
    for t in (q, k_pool, v_pool, block_table, prior_lens, k_cur, v_cur):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if block_table.dtype != torch.int32 or prior_lens.dtype != torch.int32:
        raise TypeError("block_table and prior_lens must be int32")
    for t in (q, k_pool, v_pool, k_cur, v_cur):
        if t.dtype != torch.bfloat16:
            raise TypeError("decode q, pools and current K/V must be bfloat16")
    max_blocks = block_table.shape[1]
    need = dcp_decode_workspace_size(B, Hq, D, bs, max_blocks)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _lib.call("dcp_decode_partial_active", _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(prior_lens),
              _ptr(k_cur), _ptr(v_cur), int(rank), int(world), int(interleave), B, Hq, Hkv, D, bs, max_blocks, NB,
              _scale(scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
              _stream(stream))
    return out, lse


def segmented_attention_workspace_size(Hq, Hkv, S, D, prior_tokens) -> int:
    n = ctypes.c_size_t(0)
    _lib.call("segmented_attention_workspace_size", Hq, Hkv, S, D, int(prior_tokens), ctypes.byref(n))
    return int(n.value)


def segmented_attention_partial(q, k_cur, v_cur, k_cache, v_cache, block_table, prior_tokens, rank, world,
                                interleave=16, scale=None, out=None, lse=None, workspace=None, stream=None):
    """One rank's DCP prefill partial. q [1, S, Hq, D] bf16 (the chunk's queries in global
    order); k_cur, v_cur [1, S/world, Hkv, D] bf16 (the rank's slice); k_cache [NB, Hkv, 16, D]
    and v_cache [NB, Hkv, D, 16] bf16 (the prior cache); block_table [max_blocks] int32;
    prior_tokens: the rank's prior slots. Returns (o [Hq, S, D] fp32, lse [Hq, S] fp32)."""
    _check_cuda(q, k_cur, v_cur, k_cache, v_cache, block_table, out, lse, workspace)
    _, S, Hq, D = q.shape
    _, S_local, Hkv, _ = k_cur.shape
    if k_cur.shape != v_cur.shape or k_cur.stride() != v_cur.stride():
        raise ValueError("k_cur and v_cur must share shape and strides")
    NB = k_cache.shape[0]
    if tuple(k_cache.shape) != (NB, Hkv, 16, D) or tuple(v_cache.shape) != (NB, Hkv, D, 16):
        raise ValueError("caches must be [NB, Hkv, 16, D] (K) and [NB, Hkv, D, 16] (V)")
    for t in (k_cache, v_cache, block_table):
        if not t.is_contiguous():
            raise ValueError("caches and block_table must be contiguous")
    if block_table.dtype != torch.int32:
        raise TypeError("block_table must be int32")
    need = segmented_attention_workspace_size(Hq, Hkv, S, D, prior_tokens)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((Hq, S, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((Hq, S), dtype=torch.float32, device=q.device)
    _lib.call("segmented_attention_partial", _ptr(q), _strides(q), _ptr(k_cur), _ptr(v_cur), _strides(k_cur),
              _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.numel(), NB, int(prior_tokens), int(rank),
              int(world), int(interleave), Hq, Hkv, S, S_local, D, _scale(scale), _ptr(out), _ptr(lse),
              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return out, lse


def kv_chunk_copy(dst_k, dst_v, src_k, src_v, stream=None):
    """Asynchronous device copy of one K and one V chunk (the ring hop on one GPU)."""
    _check_cuda(dst_k, dst_v, src_k, src_v)
    nbytes = src_k.numel() * src_k.element_size()
    for t in (dst_k, dst_v, src_v):
        if t.numel() * t.element_size() != nbytes:
            raise ValueError("chunk sizes differ")
    for t in (dst_k, dst_v, src_k, src_v):
        if not t.is_contiguous():
            raise ValueError("chunks must be contiguous")
    _lib.call("kv_chunk_copy", _ptr(dst_k), _ptr(dst_v), _ptr(src_k), _ptr(src_v), nbytes, _stream(stream))


def version() -> str:
    return _lib.load().ca_version().decode()
