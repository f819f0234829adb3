"""Sequence sharding rules: contiguous and striped rings, DCP interleaving.

TEST INFRASTRUCTURE ONLY (see the package docstring). Integer arithmetic, written
from the rules as the pages state them.
"""

import numpy as np


def contiguous_tokens(S: int, cp: int, rank: int) -> np.ndarray:
    """Rank r owns tokens [r*S/cp, (r+1)*S/cp) (context-parallelism page, sequence
    sharding: local_S = S // cp_size, start = cp_rank * local_S; S % cp must be 0)."""
    if S % cp:
        raise ValueError(f"sequence length {S} is not divisible by cp {cp}")
    n = S // cp
    return np.arange(rank * n, (rank + 1) * n, dtype=np.int64)


def striped_tokens(S: int, cp: int, rank: int) -> np.ndarray:
    """Striped Attention (sequence-sharding survey page): token t goes to rank t mod cp,
    so rank r's local index i holds global token i*cp + r."""
    if S % cp:
        raise ValueError(f"sequence length {S} is not divisible by cp {cp}")
    return np.arange(rank, S, cp, dtype=np.int64)


def ring_source_rank(rank: int, step: int, cp: int) -> int:
    """Whose K/V chunk rank r holds at ring step s: rank r - s (mod cp). Each rank sends
    to the next one, step 0 uses the own chunk (kernel reference page, Overview)."""
    return (rank - step) % cp


def causal_allowed(q_pos, k_pos) -> np.ndarray:
    """Causal visibility on global positions: key visible iff k_pos <= q_pos."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    return q_pos[:, None] >= k_pos[None, :]


def dcp_shard_of_position(pos, interleave: int, world: int):
    """DCP slot mapping: position p belongs to rank (p // I) % W (DCP page, slot mapping:
    blocks of I tokens dealt round-robin, e.g. I=16, W=4: block 4 wraps to rank 0)."""
    return (np.asarray(pos, dtype=np.int64) // interleave) % world


def dcp_local_filled(N: int, rank: int, block_size: int, interleave: int, world: int) -> int:
    """Tokens among positions [0, N) that rank R's shard holds: the DCP page's
    local_filled computation, step by step in its own terms."""
    vblock = block_size * world
    stride = interleave * world
    rank_start = rank * interleave
    filled = (N // vblock) * block_size
    remaining = N - (N // vblock) * vblock
    filled += (remaining // stride) * interleave
    leftover = remaining - (remaining // stride) * stride
    filled += min(max(leftover - rank_start, 0), interleave)
    return int(filled)


def dcp_active_owner(N: int, block_size: int, interleave: int, world: int) -> int:
    """The rank that owns decode position N (DCP page, dcp_active_mask)."""
    vblock = block_size * world
    pos_in_vblock = N - (N // vblock) * vblock
    return int((pos_in_vblock // interleave) % world)


def dcp_prefill_prior_global_position(slot, rank: int, interleave: int, world: int):
    """Global position of rank R's prior-cache slot s in DCP prefill (DCP page, segmented
    attention algorithm step 3): (s // I) * (W * I) + R * I + (s % I)."""
    s = np.asarray(slot, dtype=np.int64)
    return (s // interleave) * (world * interleave) + rank * interleave + (s % interleave)
