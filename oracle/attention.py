"""Plain fp64 softmax attention, LSE merge and the const-max emulation.

TEST INFRASTRUCTURE ONLY (see the package docstring). Inputs are decoded exactly
to float64; every formula below is the textbook definition, written out with no
blocking, fusion or reordering beyond row chunking to bound memory.
"""

import math

import numpy as np

# Row floor of the const-max normalisation: the kernel reference page clamps the
# row sum to 1e-37 (near the smallest fp32 normal) before the one division.
SUM_CLAMP = 1e-37
_ROW_CHUNK = 512


def to_f64(x) -> np.ndarray:
    """Exact decode to float64 (bf16 and fp32 are subsets of fp64)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def default_scale(head_dim: int) -> float:
    """softmax_scale defaults to 1/sqrt(d) (kernel reference page, Interface table)."""
    return 1.0 / math.sqrt(head_dim)


def attention(q, k, v, scale, allowed=None):
    """Softmax attention of one head with the per-row log-sum-exp.

    q [Sq, D], k [Sk, D], v [Sk, Dv]; ``allowed`` is an optional bool [Sq, Sk]
    (True = key visible to the query). Returns (O [Sq, Dv], lse [Sq]) with

        s_ij  = scale * sum_d q_id k_jd
        lse_i = log sum_{j allowed} exp(s_ij)          (natural log)
        O_i   = sum_{j allowed} exp(s_ij - lse_i) v_j

    A row with no visible key has lse = -inf and O = 0.
    """
    q = to_f64(q)
    k = to_f64(k)
    v = to_f64(v)
    Sq, Sk, Dv = q.shape[0], k.shape[0], v.shape[1]
    o = np.zeros((Sq, Dv))
    lse = np.full(Sq, -np.inf)
    if Sk == 0 or Sq == 0:
        return o, lse
    for r0 in range(0, Sq, _ROW_CHUNK):
        r1 = min(Sq, r0 + _ROW_CHUNK)
        s = scale * (q[r0:r1] @ k.T)
        if allowed is not None:
            s = np.where(np.asarray(allowed[r0:r1], dtype=bool), s, -np.inf)
        m = s.max(axis=1)
        live = np.isfinite(m)
        m_safe = np.where(live, m, 0.0)
        e = np.exp(s - m_safe[:, None])            # exp(-inf) = 0 for hidden keys
        z = e.sum(axis=1)
        row_lse = np.where(live, m_safe + np.log(np.where(live, z, 1.0)), -np.inf)
        p = np.where(live[:, None], e / np.where(live, z, 1.0)[:, None], 0.0)
        o[r0:r1] = p @ v
        lse[r0:r1] = row_lse
    return o, lse


def attention_heads(q, k, v, scale, allowed=None, kv_head_of=None):
    """``attention`` for every (batch, head) of [B, Sq, H, D] / [B, Sk, Hkv, D] tensors.

    ``kv_head_of(h)`` maps a query head to its K/V head (default: same head).
    ``allowed`` is one bool [Sq, Sk] shared by all heads, or None.
    Returns O [B, H, Sq, D] and lse [B, H, Sq].
    """
    q = to_f64(q)
    k = to_f64(k)
    v = to_f64(v)
    B, Sq, H, _ = q.shape
    Dv = v.shape[3]
    o = np.zeros((B, H, Sq, Dv))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            hk = h if kv_head_of is None else kv_head_of(h)
            o[b, h], lse[b, h] = attention(q[b, :, h], k[b, :, hk], v[b, :, hk], scale, allowed)
    return o, lse


def merge_lse(o_parts, lse_parts):
    """LSE-corrected merge of partial attention results (DCP page, decode steps 4-7).

    o_parts: sequence of n arrays [..., D]; lse_parts: n arrays [...].
        global_lse = log sum_s exp(lse_s)
        w_s        = exp(lse_s - global_lse)
        O          = sum_s w_s * O_s
    Partials with lse = -inf weigh 0; if every partial is -inf the result is
    (O = 0, lse = -inf).
    """
    L = np.stack([to_f64(x) for x in lse_parts], 0)
    O = np.stack([to_f64(x) for x in o_parts], 0)
    M = L.max(axis=0)
    live = np.isfinite(M)
    M_safe = np.where(live, M, 0.0)
    total = np.exp(L - M_safe).sum(axis=0)
    g = np.where(live, M_safe + np.log(np.where(live, total, 1.0)), -np.inf)
    w = np.where(live, np.exp(L - np.where(live, g, 0.0)), 0.0)
    out = (w[..., None] * O).sum(axis=0)
    return out, g


def const_max_bound(q, k_chunks, scale):
    """Per-row bound c_i = scale * |q_i| * max over every chunk and key of |k_j|.

    q [Sq, D]; k_chunks: iterable of [Sk_c, D]. Returns (c [Sq], kmax_sq) where
    kmax_sq = max_j |k_j|^2 over the whole ring (the all_reduce(max) of the page).
    """
    q = to_f64(q)
    kmax_sq = 0.0
    for kc in k_chunks:
        kc = to_f64(kc)
        if kc.shape[0]:
            kmax_sq = max(kmax_sq, float((kc * kc).sum(axis=1).max()))
    qn = np.sqrt((q * q).sum(axis=1))
    return scale * qn * math.sqrt(kmax_sq), kmax_sq


def const_max(q, k_chunks, v_chunks, scale, clamp=SUM_CLAMP):
    """The const-max ring method of the kernel reference page, in fp64.

    Step 0 initialises and every later step adds (no rescale):
        Z_i += sum_j exp(s_ij - c_i),   A_i += sum_j exp(s_ij - c_i) v_j
    then once:  O_i = A_i / max(Z_i, clamp),  lse_i = c_i + log(max(Z_i, clamp)).
    Returns (O [Sq, Dv], lse [Sq], c [Sq]).

    In exact arithmetic this equals ``attention`` (softmax is shift invariant); it
    departs only when the bound overshoots a row's largest score by about
    -log(clamp) = 85.2 nats, where the clamp takes over (the page's documented
    failure mode).
    """
    q = to_f64(q)
    k_chunks = [to_f64(x) for x in k_chunks]
    v_chunks = [to_f64(x) for x in v_chunks]
    c, _ = const_max_bound(q, k_chunks, scale)
    Dv = v_chunks[0].shape[1]
    Z = np.zeros(q.shape[0])
    A = np.zeros((q.shape[0], Dv))
    for kc, vc in zip(k_chunks, v_chunks):
        if kc.shape[0] == 0:
            continue
        for r0 in range(0, q.shape[0], _ROW_CHUNK):
            r1 = min(q.shape[0], r0 + _ROW_CHUNK)
            p = np.exp(scale * (q[r0:r1] @ kc.T) - c[r0:r1, None])
            Z[r0:r1] += p.sum(axis=1)
            A[r0:r1] += p @ vc
    Zc = np.maximum(Z, clamp)
    return A / Zc[:, None], c + np.log(Zc), c


def key_sinks(k_chunks, theta, max_sinks):
    """Sink keys of the ring: |k_j| above theta times the mean key norm over every chunk
    (kernel reference page, "Adapting this kernel": a handful of keys whose norms dwarf the
    rest inflate max_j |k_j| for every row; excluding them from the max recovers the bound).
    The mean of the norms, not of their squares, so that a few sinks 100-1000x louder than
    the rest barely move the reference. More than ``max_sinks`` such keys, or theta <= 0,
    means no exclusion. Returns one bool mask per chunk."""
    k_chunks = [to_f64(x) for x in k_chunks]
    norms = [np.sqrt((kc * kc).sum(axis=1)) for kc in k_chunks]
    total = sum(int(n.shape[0]) for n in norms)
    if theta <= 0 or total == 0:
        return [np.zeros(n.shape[0], dtype=bool) for n in norms]
    mean = sum(float(n.sum()) for n in norms) / total
    masks = [n > theta * mean for n in norms]
    if sum(int(m.sum()) for m in masks) > max_sinks:
        return [np.zeros(n.shape[0], dtype=bool) for n in norms]
    return masks


def const_max_sink_robust(q, k_chunks, v_chunks, scale, theta, max_sinks, clamp=SUM_CLAMP):
    """Const-max with the sinks taken out of the bound: the bound c_i uses the largest
    non-sink key norm, the const-max fold runs over the non-sink keys, the sink keys are
    attended exactly on their own, and the two partials are merged by the LSE rule.
    Returns (O [Sq, Dv], lse [Sq], c [Sq]). In exact arithmetic this is ``attention``."""
    q = to_f64(q)
    k_chunks = [to_f64(x) for x in k_chunks]
    v_chunks = [to_f64(x) for x in v_chunks]
    masks = key_sinks(k_chunks, theta, max_sinks)
    kn = [kc[~m] for kc, m in zip(k_chunks, masks)]
    vn = [vc[~m] for vc, m in zip(v_chunks, masks)]
    ks = np.concatenate([kc[m] for kc, m in zip(k_chunks, masks)], axis=0)
    vs = np.concatenate([vc[m] for vc, m in zip(v_chunks, masks)], axis=0)
    Dv = v_chunks[0].shape[1]
    if sum(x.shape[0] for x in kn):
        o_n, lse_n, c = const_max(q, kn, vn, scale, clamp)
    else:
        o_n, lse_n, c = np.zeros((q.shape[0], Dv)), np.full(q.shape[0], -np.inf), np.zeros(q.shape[0])
    o_s, lse_s = attention(q, ks, vs, scale)
    o, lse = merge_lse([o_n, o_s], [lse_n, lse_s])
    return o, lse, c
