"""Host-side logic of the product (ring schedule, shard views, step masks, DCP cache
building) against the oracle's independent statement of the same rules (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from context_attention_lse_amd import dcp as cdcp
from context_attention_lse_amd import ring


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_ring_schedule_matches_oracle(cp):
    for r in range(cp):
        for s in range(cp):
            assert ring.ring_source_rank(r, s, cp) == oracle.ring_source_rank(r, s, cp)


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_shard_views_hold_the_oracle_tokens(layout):
    S, cp = 48, 4
    x = torch.arange(S).reshape(1, S, 1, 1).expand(1, S, 2, 8).contiguous()
    fn = oracle.contiguous_tokens if layout == "contiguous" else oracle.striped_tokens
    pool = ring.chunk_pool(x, cp, layout)
    for r in range(cp):
        got = ring.shard(x, cp, r, layout)[0, :, 0, 0].numpy()
        assert np.array_equal(got, fn(S, cp, r))
        assert np.array_equal(pool[r, 0, :, 0, 0].numpy(), fn(S, cp, r))


def test_indivisible_sequence_is_rejected_like_the_page_example():
    x = torch.zeros((1, 3645, 1, 8))
    with pytest.raises(ValueError, match="3645 is not divisible by cp_size 8"):
        ring.shard(x, 8, 0, "contiguous")


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
@pytest.mark.parametrize("cp", [2, 4, 8])
def test_step_masks_equal_global_causality(layout, cp):
    """The per-step local mask the driver picks reproduces causality on global positions."""
    L = 6
    S = L * cp
    fn = oracle.contiguous_tokens if layout == "contiguous" else oracle.striped_tokens
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    local = {"none": np.ones((L, L), bool), "causal_incl": j <= i, "causal_strict": j < i, None: np.zeros((L, L), bool)}
    for r in range(cp):
        for s in range(cp):
            src = ring.ring_source_rank(r, s, cp)
            want = oracle.causal_allowed(fn(S, cp, r), fn(S, cp, src))
            got = local[ring.step_mask(layout, True, r, src)]
            assert np.array_equal(got, want), (layout, r, s)
        assert ring.step_mask(layout, False, r, (r + 1) % cp) == "none"


def test_local_filled_matches_page_formula():
    for W in (1, 2, 4, 8):
        for N in range(0, 600):
            for r in range(W):
                assert cdcp.local_filled(N, r, 16, W) == oracle.dcp_local_filled(N, r, 16, 16, W)


def test_shard_positions_are_the_shard():
    for W in (2, 4):
        for N in (0, 7, 16, 33, 500):
            for r in range(W):
                want = np.nonzero(oracle.dcp_shard_of_position(np.arange(N), 16, W) == r)[0]
                assert np.array_equal(cdcp.shard_positions(N, r, 16, W), want)


def test_build_shard_cache_places_every_token():
    torch.manual_seed(0)
    ctx = np.array([5, 40, 100])
    offsets = np.concatenate([[0], np.cumsum(ctx)])
    Hkv, D = 2, 8
    k = torch.randn((int(offsets[-1]), Hkv, D))
    v = torch.randn((int(offsets[-1]), Hkv, D))
    rand = np.random.default_rng(1).random(64)
    for r in range(2):
        sc = cdcp.build_shard_cache(k, v, offsets, ctx, r, 2, 16, 16, rand)
        for b in range(3):
            pos = cdcp.shard_positions(int(ctx[b]), r, 16, 2)
            assert int(sc.local_lens[b]) == len(pos)
            for t, p in enumerate(pos):
                blk = int(sc.block_table[b, t // 16])
                assert torch.equal(sc.k_pool[blk, :, t % 16, :], k[offsets[b] + p])
                assert torch.equal(sc.v_pool[blk, :, :, t % 16], v[offsets[b] + p])
        used = [int(sc.block_table[b, j]) for b in range(3) for j in range(-(-int(sc.local_lens[b]) // 16))]
        assert len(set(used)) == len(used)   # physical blocks are distinct
