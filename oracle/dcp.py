"""DCP decode in fp64: one shard's partial attention, and full attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

DCP page, decode compute pattern: the gathered query attends the rank's local KV
shard (the positions whose interleave block maps to that rank) and returns a
partial output with its LSE; the partials are merged by ``attention.merge_lse``.
Query head h reads K/V head h // (Hq / Hkv) (contiguous GQA groups; the pages do
not fix the grouping, this is the plain reading).
"""

import numpy as np

from .attention import attention, to_f64
from .sharding import (causal_allowed, dcp_active_owner, dcp_prefill_prior_global_position,
                       dcp_shard_of_position)


def decode_shard_partial(q, k_seq, v_seq, rank: int, interleave: int, world: int, scale):
    """q [Hq, D]; k_seq, v_seq [N, Hkv, D] in token order. Returns (O [Hq, D], lse [Hq])
    over the tokens of shard ``rank`` only."""
    q = to_f64(q)
    k_seq = to_f64(k_seq)
    v_seq = to_f64(v_seq)
    N = k_seq.shape[0]
    mine = dcp_shard_of_position(np.arange(N), interleave, world) == rank
    return _decode(q, k_seq[mine], v_seq[mine], scale)


def decode_shard_partial_active(q, k_prior, v_prior, k_act, v_act, rank: int, interleave: int, world: int,
                                block_size: int, scale):
    """One shard's decode partial with the page's two-part mask (DCP page, active token
    handling and dcp_active_mask): the prior positions [0, N) that this rank holds, plus
    the current token at position N only on the rank that owns N, so that the merged
    result counts it once. k_prior, v_prior [N, Hkv, D]; k_act, v_act [Hkv, D]."""
    q = to_f64(q)
    k_prior = to_f64(k_prior)
    v_prior = to_f64(v_prior)
    N = k_prior.shape[0]
    mine = dcp_shard_of_position(np.arange(N), interleave, world) == rank
    k = k_prior[mine]
    v = v_prior[mine]
    if dcp_active_owner(N, block_size, interleave, world) == rank:
        k = np.concatenate([k, to_f64(k_act)[None]], axis=0)
        v = np.concatenate([v, to_f64(v_act)[None]], axis=0)
    return _decode(q, k, v, scale)


def decode_full(q, k_seq, v_seq, scale):
    """Attention of the decode token against the whole sequence (no sharding)."""
    return _decode(to_f64(q), to_f64(k_seq), to_f64(v_seq), scale)


def _decode(q, k, v, scale):
    Hq = q.shape[0]
    Hkv = k.shape[1]
    group = Hq // Hkv
    o = np.zeros((Hq, v.shape[2]))
    lse = np.zeros(Hq)
    for h in range(Hq):
        hk = h // group
        oh, lh = attention(q[h:h + 1], k[:, hk], v[:, hk], scale)
        o[h], lse[h] = oh[0], lh[0]
    return o, lse


def segmented_attention_partial(q, k_cur, v_cur, k_prior, v_prior, prior_global: int, rank: int,
                                interleave: int, world: int, scale):
    """One rank's DCP prefill partial (DCP page, segmented attention algorithm steps 1-4).

    q [S, Hq, D]: every query of the current chunk in global order, query i at global
    position prior_global + i. k_cur, v_cur [S/W, Hkv, D]: this rank's slice of the
    chunk, local token j at prior_global + (j // I)(W I) + R I + (j % I). k_prior,
    v_prior [n, Hkv, D]: this rank's prior cache slots, slot s at
    (s // I)(W I) + R I + (s % I). A key is visible when its global position is at most
    the query's. Returns (O [Hq, S, D], lse [Hq, S]) over the prior and current keys."""
    q = to_f64(q)
    k = np.concatenate([to_f64(k_prior), to_f64(k_cur)], axis=0)
    v = np.concatenate([to_f64(v_prior), to_f64(v_cur)], axis=0)
    n_prior, n_cur = k_prior.shape[0], k_cur.shape[0]
    kpos = np.concatenate([
        dcp_prefill_prior_global_position(np.arange(n_prior), rank, interleave, world),
        prior_global + dcp_prefill_prior_global_position(np.arange(n_cur), rank, interleave, world)])
    qpos = prior_global + np.arange(q.shape[0])
    allowed = causal_allowed(qpos, kpos)
    Hq, Hkv = q.shape[1], k.shape[1]
    group = Hq // Hkv
    o = np.zeros((Hq, q.shape[0], v.shape[2]))
    lse = np.zeros((Hq, q.shape[0]))
    for h in range(Hq):
        o[h], lse[h] = attention(q[:, h], k[:, h // group], v[:, h // group], scale, allowed)
    return o, lse
