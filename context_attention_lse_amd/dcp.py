"""DCP decode on one GPU: build each shard's paged KV cache, run every shard's partial,
merge the shards by LSE.

Interleaving follows "DCP (Decode Context Parallelism)": positions are dealt to ranks in
blocks of ``interleave`` tokens round-robin (slot mapping: position p belongs to rank
(p div I) mod W), each rank keeps its tokens in order in a paged cache, and
local_filled gives how many of a context's N tokens a rank holds. A decode step runs
every rank's local attention and combines the partials with weights
exp(local_lse - global_lse) (here: lse_merge over the shards, standing in for the LSE
all-gather and output reduce-scatter).

Cache layout (this library's): K blocks [num_blocks, Hkv, block_size, D] token-major,
V blocks [num_blocks, Hkv, D, block_size] d-major; physical block ids are a seeded
shuffle, so block tables are genuinely indirect.

Building the cache is set-up work (the cache write of earlier decode steps), done with
torch indexing; the decode itself runs in libctxattn.
"""

import math

import numpy as np
import torch

from . import api


def local_filled(N: int, rank: int, interleave: int, world: int) -> int:
    """Tokens of a context of N that rank ``rank`` holds: whole rounds of interleave*world
    positions give ``interleave`` each, the partial round gives the part of the rank's
    interleave window that it reaches."""
    rnd = interleave * world
    full, rem = divmod(int(N), rnd)
    return full * interleave + min(max(rem - rank * interleave, 0), interleave)


def shard_positions(N: int, rank: int, interleave: int, world: int) -> np.ndarray:
    """Global positions of the rank's tokens, in shard-local order."""
    n = local_filled(N, rank, interleave, world)
    t = np.arange(n, dtype=np.int64)
    return (t // interleave) * (interleave * world) + rank * interleave + (t % interleave)


class ShardCache:
    """One rank's paged cache for a batch of sequences."""

    def __init__(self, k_pool, v_pool, block_table, local_lens, max_blocks):
        self.k_pool, self.v_pool = k_pool, v_pool
        self.block_table, self.local_lens = block_table, local_lens
        self.max_blocks = max_blocks

    @property
    def nbytes_kv(self) -> int:
        """Resident K+V bytes that one decode step must read."""
        Hkv, D = self.k_pool.shape[1], self.k_pool.shape[3]
        return int(self.local_lens.sum().item()) * Hkv * D * 2 * self.k_pool.element_size()


def build_shard_cache(k_seq, v_seq, offsets, ctx, rank, world, interleave=16, block_size=16,
                      block_rand=None, max_blocks=None) -> ShardCache:
    """Write rank ``rank``'s tokens of every sequence into a fresh paged cache.

    k_seq, v_seq [sum(ctx), Hkv, D] hold every sequence's tokens in order (sequence b at
    rows offsets[b] .. offsets[b+1]); block_rand: uniform draws used to shuffle physical
    block ids (identity order if None)."""
    dev = k_seq.device
    Hkv, D = k_seq.shape[1], k_seq.shape[2]
    B = len(ctx)
    lens = [local_filled(int(n), rank, interleave, world) for n in ctx]
    nblk = [math.ceil(n / block_size) for n in lens]
    total_blocks = sum(nblk)
    if max_blocks is None:
        max_blocks = max(1, max(nblk) if nblk else 1)
    if block_rand is not None:
        key = np.asarray(block_rand[rank::world][:total_blocks])
        if key.shape[0] < total_blocks:
            raise ValueError("not enough block_rand draws for this cache")
        phys = np.argsort(key, kind="stable").astype(np.int64)
    else:
        phys = np.arange(total_blocks, dtype=np.int64)
    table = np.zeros((B, max_blocks), dtype=np.int32)
    src_rows, dst_blk, dst_slot = [], [], []
    b0 = 0
    for b in range(B):
        table[b, :nblk[b]] = phys[b0:b0 + nblk[b]]
        pos = shard_positions(int(ctx[b]), rank, interleave, world)
        t = np.arange(len(pos), dtype=np.int64)
        src_rows.append(int(offsets[b]) + pos)
        dst_blk.append(phys[b0 + t // block_size])
        dst_slot.append(t % block_size)
        b0 += nblk[b]
    k_pool = torch.zeros((max(total_blocks, 1), Hkv, block_size, D), dtype=k_seq.dtype, device=dev)
    v_pool = torch.zeros((max(total_blocks, 1), Hkv, D, block_size), dtype=v_seq.dtype, device=dev)
    if total_blocks:
        src = torch.from_numpy(np.concatenate(src_rows)).to(dev)
        blk = torch.from_numpy(np.concatenate(dst_blk)).to(dev)
        slot = torch.from_numpy(np.concatenate(dst_slot)).to(dev)
        # K[blk, h, slot, :] and V[blk, h, :, slot] <- token rows
        k_pool.permute(0, 2, 1, 3)[blk, slot] = k_seq[src]
        v_pool.permute(0, 3, 1, 2)[blk, slot] = v_seq[src]
    return ShardCache(k_pool, v_pool, torch.from_numpy(table).to(dev),
                      torch.tensor(lens, dtype=torch.int32, device=dev), max_blocks)


class DcpDecode:
    """Every shard's decode partial plus the cross-shard LSE merge, with preallocated
    outputs and workspaces (one per shard) so repeated steps allocate nothing."""

    def __init__(self, q, shards, scale=None):
        self.q, self.shards, self.scale = q, list(shards), scale
        B, Hq, D = q.shape
        dev = q.device
        W = len(self.shards)
        self.o_parts = torch.empty((W, B, Hq, D), dtype=torch.float32, device=dev)
        self.lse_parts = torch.empty((W, B, Hq), dtype=torch.float32, device=dev)
        self.ws = []
        for sc in self.shards:
            need = api.dcp_decode_workspace_size(B, Hq, D, sc.k_pool.shape[2], sc.max_blocks)
            self.ws.append(torch.empty(max(need, 16), dtype=torch.uint8, device=dev))
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)

    def run(self):
        for r, sc in enumerate(self.shards):
            api.dcp_decode_partial(self.q, sc.k_pool, sc.v_pool, sc.block_table, sc.local_lens, scale=self.scale,
                                   out=self.o_parts[r], lse=self.lse_parts[r], workspace=self.ws[r])
        api.lse_merge(self.o_parts, self.lse_parts, out=self.out, lse_out=self.lse)
        return self.out, self.lse

    def run_active(self, prior_lens, k_cur, v_cur, interleave=16):
        """A decode step with the current token: the shards hold the prior tokens
        (positions [0, N) of each sequence, N = prior_lens), every shard gets the current
        token's K/V, and only the owner of position N attends it (dcp_active_mask)."""
        W = len(self.shards)
        for r, sc in enumerate(self.shards):
            api.dcp_decode_partial_active(self.q, sc.k_pool, sc.v_pool, sc.block_table, prior_lens, k_cur, v_cur,
                                          r, W, interleave, scale=self.scale, out=self.o_parts[r],
                                          lse=self.lse_parts[r], workspace=self.ws[r])
        api.lse_merge(self.o_parts, self.lse_parts, out=self.out, lse_out=self.lse)
        return self.out, self.lse


def rank_slice(x, world: int, rank: int, interleave: int):
    """Rank ``rank``'s tokens of a chunk x [1, S, H, D] in local order: the blocks of
    ``interleave`` positions that the slot mapping deals to it (S a multiple of W * I)."""
    _, S, H, D = x.shape
    if S % (world * interleave):
        raise ValueError(f"chunk length {S} is not a multiple of world * interleave = {world * interleave}")
    return x.view(S // (world * interleave), world, interleave, H, D)[:, rank].reshape(1, S // world, H, D)


class DcpPrefill:
    """DCP prefill of one chunk on one GPU: every rank's segmented attention (its prior
    cache plus its slice of the chunk), then the LSE merge over the ranks, standing in
    for the page's LSE all-gather and output reduce-scatter.

    q [1, S, Hq, D]: the chunk's queries; k_chunk, v_chunk [1, S, Hkv, D]: the chunk's
    keys/values in global order (each rank keeps only its slice); caches: one ShardCache
    per rank holding the prior tokens (batch of one sequence); prior_global: the prior
    length."""

    def __init__(self, q, k_chunk, v_chunk, caches, prior_global, interleave=16, scale=None):
        self.W = len(caches)
        self.q, self.caches, self.interleave, self.scale = q, list(caches), interleave, scale
        self.k_local = [rank_slice(k_chunk, self.W, r, interleave).contiguous() for r in range(self.W)]
        self.v_local = [rank_slice(v_chunk, self.W, r, interleave).contiguous() for r in range(self.W)]
        self.prior = [local_filled(prior_global, r, interleave, self.W) for r in range(self.W)]
        _, S, Hq, D = q.shape
        Hkv = k_chunk.shape[2]
        dev = q.device
        self.o_parts = torch.empty((self.W, Hq, S, D), dtype=torch.float32, device=dev)
        self.lse_parts = torch.empty((self.W, Hq, S), dtype=torch.float32, device=dev)
        self.ws = [torch.empty(max(16, api.segmented_attention_workspace_size(Hq, Hkv, S, D, n)), dtype=torch.uint8,
                               device=dev) for n in self.prior]
        self.out = torch.empty((Hq, S, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((Hq, S), dtype=torch.float32, device=dev)

    def run(self):
        for r, sc in enumerate(self.caches):
            api.segmented_attention_partial(self.q, self.k_local[r], self.v_local[r], sc.k_pool, sc.v_pool,
                                            sc.block_table[0], self.prior[r], r, self.W, self.interleave,
                                            scale=self.scale, out=self.o_parts[r], lse=self.lse_parts[r],
                                            workspace=self.ws[r])
        api.lse_merge(self.o_parts, self.lse_parts, out=self.out, lse_out=self.lse)
        return self.out, self.lse
