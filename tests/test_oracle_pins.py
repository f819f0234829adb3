"""The fp64 oracle against brute force, closed forms, invariants and the pages'
printed examples (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import oracle

from pins import (brute_attention, pins_attention, pins_const_max, pins_dcp_active, pins_merge, pins_segmented,
                  pins_sink_robust)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_attention_pinned():
    assert pins_attention(oracle.attention) == []


def test_merge_pinned():
    assert pins_merge(oracle.attention, oracle.merge_lse) == []


def test_const_max_pinned():
    assert pins_const_max(oracle.attention, oracle.const_max, oracle.const_max_bound) == []


def test_default_scale():
    assert oracle.default_scale(128) == 1.0 / math.sqrt(128.0)
    assert oracle.default_scale(64) == 0.125


def test_attention_heads_matches_brute_force_gqa():
    rng = np.random.default_rng(3)
    B, Sq, Sk, H, Hkv, D = 2, 3, 5, 4, 2, 3
    q = rng.normal(size=(B, Sq, H, D)); k = rng.normal(size=(B, Sk, Hkv, D)); v = rng.normal(size=(B, Sk, Hkv, 2))
    o, l = oracle.attention_heads(q, k, v, 0.5, kv_head_of=lambda h: h // 2)
    for b in range(B):
        for h in range(H):
            bo, bl = brute_attention(q[b, :, h], k[b, :, h // 2], v[b, :, h // 2], 0.5)
            assert np.allclose(o[b, h], bo, atol=1e-13) and np.allclose(l[b, h], bl, atol=1e-13)


def test_bf16_decode_is_exact():
    torch = pytest.importorskip("torch")
    x = torch.randn(1000).to(torch.bfloat16)
    y = oracle.to_f64(x)
    # bf16 -> fp64 is exact: every value survives a round trip back through bf16
    assert torch.equal(torch.from_numpy(y).to(torch.bfloat16), x)
    assert np.array_equal(y, x.float().double().numpy())


# ---------------------------------------------------------------- sharding rules

def test_dcp_slot_mapping_example():
    g = _golden("dcp_slot_mapping.json")
    for blk in g["blocks"]:
        pos = np.arange(blk["first"], blk["last"] + 1)
        ranks = oracle.dcp_shard_of_position(pos, g["interleave"], g["world"])
        assert np.all(ranks == blk["rank"]), blk
    for world, key in ((4, "rank_blocks_world4"), (2, "rank_blocks_world2")):
        for rank, blocks in g[key].items():
            for b in blocks:
                pos = np.arange(16 * b, 16 * b + 16)
                assert np.all(oracle.dcp_shard_of_position(pos, 16, world) == int(rank))


@pytest.mark.parametrize("world", [1, 2, 4, 8])
@pytest.mark.parametrize("interleave,block_size", [(1, 1), (4, 4), (8, 16), (16, 16), (16, 32)])
def test_dcp_local_filled_brute_force(world, interleave, block_size):
    for N in range(0, 700):
        shard = oracle.dcp_shard_of_position(np.arange(N), interleave, world)
        for r in range(world):
            assert oracle.dcp_local_filled(N, r, block_size, interleave, world) == int(np.sum(shard == r)), (N, r)


def test_dcp_local_filled_partitions_every_length():
    for N in (0, 1, 15, 16, 17, 31, 32, 33, 32768, 131071, 131072):
        assert sum(oracle.dcp_local_filled(N, r, 16, 16, 2) for r in range(2)) == N


def test_dcp_active_owner_is_the_position_owner():
    for world in (1, 2, 4):
        for N in range(0, 300):
            assert oracle.dcp_active_owner(N, 16, 16, world) == int(oracle.dcp_shard_of_position(N, 16, world))


def test_dcp_prefill_prior_positions_enumerate_the_shard():
    for world in (2, 4):
        for rank in range(world):
            n = oracle.dcp_local_filled(1000, rank, 16, 16, world)
            got = oracle.dcp_prefill_prior_global_position(np.arange(n), rank, 16, world)
            want = np.nonzero(oracle.dcp_shard_of_position(np.arange(1000), 16, world) == rank)[0]
            assert np.array_equal(got, want)


def test_sequence_divisibility_example():
    g = _golden("wan_sequence_divisibility.json")
    assert g["latent_frames"] * g["post_patch_h"] * g["post_patch_w"] == g["S_total"]
    assert g["S_total"] % g["cp"] == g["remainder"]
    with pytest.raises(ValueError):
        oracle.contiguous_tokens(g["S_total"], g["cp"], 0)
    with pytest.raises(ValueError):
        oracle.striped_tokens(g["S_total"], g["cp"], 0)


def test_ring_schedule_example():
    g = _golden("ring_schedule_cp4.json")
    for r, row in enumerate(g["chunk_at_step"]):
        assert [oracle.ring_source_rank(r, s, g["cp"]) for s in range(g["cp"])] == row


@pytest.mark.parametrize("cp", [1, 2, 3, 8])
def test_shardings_partition_the_sequence(cp):
    S = 24 * cp
    for fn in (oracle.contiguous_tokens, oracle.striped_tokens):
        allt = np.concatenate([fn(S, cp, r) for r in range(cp)])
        assert np.array_equal(np.sort(allt), np.arange(S))
    assert np.array_equal(oracle.striped_tokens(S, cp, cp - 1), np.arange(cp - 1, S, cp))


# ---------------------------------------------------------------- composed cases

def test_striped_causal_ring_equals_full_causal():
    rng = np.random.default_rng(5)
    S, cp, D = 32, 4, 4
    q = rng.normal(size=(S, D)); k = rng.normal(size=(S, D)); v = rng.normal(size=(S, 3))
    full_o, full_l = oracle.attention(q, k, v, 0.5, oracle.causal_allowed(np.arange(S), np.arange(S)))
    for r in range(cp):
        tq = oracle.striped_tokens(S, cp, r)
        parts = []
        for s in range(cp):
            tk = oracle.striped_tokens(S, cp, oracle.ring_source_rank(r, s, cp))
            parts.append(oracle.attention(q[tq], k[tk], v[tk], 0.5, oracle.causal_allowed(tq, tk)))
        o, l = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(o, full_o[tq], atol=1e-12) and np.allclose(l, full_l[tq], atol=1e-12)


def test_contiguous_ring_const_max_equals_full():
    rng = np.random.default_rng(6)
    S, cp, D = 40, 4, 8
    q = rng.normal(size=(S, D)); k = rng.normal(size=(S, D)); v = rng.normal(size=(S, 3))
    full_o, full_l = oracle.attention(q, k, v, 0.3)
    for r in range(cp):
        tq = oracle.contiguous_tokens(S, cp, r)
        order = [oracle.contiguous_tokens(S, cp, oracle.ring_source_rank(r, s, cp)) for s in range(cp)]
        o, l, c = oracle.const_max(q[tq], [k[t] for t in order], [v[t] for t in order], 0.3)
        assert np.allclose(o, full_o[tq], atol=1e-12) and np.allclose(l, full_l[tq], atol=1e-12)
        assert np.all(c >= full_l[tq] - math.log(S))   # c bounds every score, so lse <= c + log S


@pytest.mark.parametrize("N", [1, 9, 16, 17, 40, 75])
def test_dcp_decode_shards_merge_to_full(N):
    rng = np.random.default_rng(N)
    Hq, Hkv, D = 4, 2, 3
    q = rng.normal(size=(Hq, D)) * 2; k = rng.normal(size=(N, Hkv, D)); v = rng.normal(size=(N, Hkv, 2))
    parts = [oracle.decode_shard_partial(q, k, v, r, 16, 2, 0.5) for r in range(2)]
    o, l = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts])
    fo, fl = oracle.decode_full(q, k, v, 0.5)
    assert np.allclose(o, fo, atol=1e-12) and np.allclose(l, fl, atol=1e-12)
    if N <= 16:
        assert np.all(parts[1][1] == -np.inf) and np.all(parts[1][0] == 0)
    # each shard partial by brute force over its own tokens
    for r in range(2):
        mine = [p for p in range(N) if (p // 16) % 2 == r]
        for h in range(Hq):
            bo, bl = brute_attention(q[h:h + 1], k[mine, h // 2], v[mine, h // 2], 0.5)
            assert np.allclose(parts[r][0][h], bo[0], atol=1e-12)
            assert (parts[r][1][h] == bl[0]) or abs(parts[r][1][h] - bl[0]) < 1e-12


@pytest.mark.parametrize("world", [1, 2, 3, 4])
@pytest.mark.parametrize("interleave", [1, 4, 16])
def test_dcp_decode_active_token_counts_once(world, interleave):
    assert pins_dcp_active(oracle.decode_shard_partial_active, world, interleave) == []


def test_dcp_decode_ungated_active_token_is_not_full_attention():
    """Without the gate every rank adds the current token and the merge weighs it W times."""
    Hq, Hkv, D = 2, 1, 3
    q = np.ones((Hq, D)); k = np.zeros((5, Hkv, D)); v = np.zeros((5, Hkv, 2))
    ka = np.ones((Hkv, D)); va = np.ones((Hkv, 2))
    parts = []
    for r in range(2):
        mine = [p for p in range(5) if (p // 1) % 2 == r]
        parts.append(oracle.decode_full(q, np.concatenate([k[mine], ka[None]]), np.concatenate([v[mine], va[None]]), 0.5))
    o, _ = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts])
    fo, _ = oracle.decode_full(q, np.concatenate([k, ka[None]]), np.concatenate([v, va[None]]), 0.5)
    assert not np.allclose(o, fo, atol=1e-6)


@pytest.mark.parametrize("world,interleave", [(1, 16), (2, 1), (2, 4), (2, 16), (4, 4), (3, 2)])
@pytest.mark.parametrize("prior_rounds", [0, 1, 3])
def test_dcp_prefill_segments_merge_to_causal_attention(world, interleave, prior_rounds):
    assert pins_segmented(oracle.segmented_attention_partial, world, interleave, prior_rounds) == []


def test_sink_robust_const_max_pinned():
    assert pins_sink_robust(oracle.const_max_sink_robust, oracle.key_sinks) == []


def test_plain_const_max_collapses_on_the_sink_pin_input():
    """The input of the sink pins defeats the plain bound: rows collapse (the page's named
    failure), so the robust result above is not the plain one by accident."""
    rng = np.random.default_rng(29)
    q = rng.normal(size=(7, 8)) * 3.0
    ks = [rng.normal(size=(6, 8)) for _ in range(3)]
    vs = [rng.normal(size=(6, 3)) for _ in range(3)]
    ks[0][4] *= 60.0
    ks[2][1] = -ks[2][1] * 45.0
    o, l, _ = oracle.const_max(q, ks, vs, 0.5)
    eo, el = oracle.attention(q, np.concatenate(ks), np.concatenate(vs), 0.5)
    assert np.abs(l - el).max() > 1.0


def test_sum_clamp_value():
    assert oracle.SUM_CLAMP == 1e-37
    assert abs(-math.log(oracle.SUM_CLAMP) - 85.2) < 0.1   # the page's ~85 nats
