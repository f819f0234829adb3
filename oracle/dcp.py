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
from .sharding import dcp_shard_of_position


def decode_shard_partial(q, k_seq, v_seq, rank: int, interleave: int, world: int, scale):
    """q [Hq, D]; k_seq, v_seq [N, Hkv, D] in token order. Returns (O [Hq, D], lse [Hq])
    over the tokens of shard ``rank`` only."""
    q = to_f64(q)
    k_seq = to_f64(k_seq)
    v_seq = to_f64(v_seq)
    N = k_seq.shape[0]
    mine = dcp_shard_of_position(np.arange(N), interleave, world) == rank
    return _decode(q, k_seq[mine], v_seq[mine], scale)


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
