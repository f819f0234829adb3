"""HIP path vs the fp64 oracle at the workloads' full sizes, in the launch configuration the
benchmark times (RingPass / DcpDecode with their defaults), on sampled output rows that the
oracle computes one by one against the full key range.

Rows are sampled per head with a fixed seed and always include the first rows, both sides of
the 256-row query-tile edges, the ragged last tile and the last row; every sampled row is
checked element by element."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check, say
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ca():
    import context_attention_lse_amd as ca
    ca._lib.load()
    torch.cuda.set_device(0)
    return ca


def _rows(n, seed, k=24):
    last_tile = (n - 1) // 256 * 256
    return gen.sample_rows(n, k, seed, include=(0, 1, 255, 256, last_tile - 1, last_tile, n - 2, n - 1))


def _ring_fullsize(ca, name, variant, rank, heads, contiguous_q, **ring_kw):
    wl = workloads.workload(name)
    dev = torch.device("cuda:0")
    say(f"full-size {name} variant={variant} rank={rank} S={wl.S} cp={wl.cp} H={wl.H} {ring_kw}")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, rank, wl.layout)
    if contiguous_q:
        q = q.contiguous()
    kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
    rp = ca.ring.RingPass(q, kp, vp, rank, layout=wl.layout, causal=wl.causal, variant=variant, **ring_kw)
    o, lse = rp.run()
    torch.cuda.synchronize()
    tok = (oracle.contiguous_tokens if wl.layout == "contiguous" else oracle.striped_tokens)(wl.S, wl.cp, rank)
    scale = oracle.default_scale(wl.D)
    for h in heads:
        rows = _rows(wl.local_S, 17 * h + rank)
        qh = oracle.to_f64(t["q"][0, tok[rows], h])
        kh = oracle.to_f64(t["k"][0, :, h])
        vh = oracle.to_f64(t["v"][0, :, h])
        allowed = oracle.causal_allowed(tok[rows], np.arange(wl.S)) if wl.causal else None
        ro, rl = oracle.attention(qh, kh, vh, scale, allowed)
        check(f"{name} {variant} rank {rank} head {h} ({len(rows)} rows)", o[0, h, rows], lse[0, h, rows], ro, rl)
    del t, q, kp, vp, rp
    torch.cuda.empty_cache()


def test_wan22_cp8_online_fullsize(ca):
    # the headline's launch configuration: key-split steps alternating two compute streams,
    # each carrying the hop of the chunk two steps ahead
    _ring_fullsize(ca, "wan22_cp8_online", "online", 0, heads=(0, 4, 9), contiguous_q=False, split=True,
                   compute_streams=2, fused_hops=True)


def test_wan22_cp8_online_fullsize_copy_stream(ca):
    # the same with the hops on a copy stream
    _ring_fullsize(ca, "wan22_cp8_online", "online", 3, heads=(1, 8), contiguous_q=False, split=True,
                   compute_streams=2)


def test_wan22_cp8_online_fullsize_unsplit(ca):
    _ring_fullsize(ca, "wan22_cp8_online", "online", 5, heads=(2, 7), contiguous_q=False)


def test_wan22_720p_constmax_sinks_fullsize(ca):
    """The sink-robust pass as timed (theta 4): exact attention is the target whether or not
    any key qualifies as a sink."""
    _ring_fullsize(ca, "wan22_720p_constmax", "constmax", 0, heads=(0, 39), contiguous_q=True, sink_theta=4.0)


@pytest.mark.parametrize("variant", ["constmax", "online"])
def test_wan22_720p_fullsize(ca, variant):
    # the bench's launch configurations: const-max steps carry their hops, online ones do not
    _ring_fullsize(ca, "wan22_720p_constmax", variant, 0, heads=(0, 21, 39), contiguous_q=True,
                   fused_hops=(variant == "constmax"))


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_striped_causal_128k_fullsize(ca, rank):
    _ring_fullsize(ca, "striped_causal_128k", "online", rank, heads=(0, 31), contiguous_q=True)


def test_dcp_decode_fullsize(ca):
    wl = workloads.workload("dcp_decode_gqa")
    dev = torch.device("cuda:0")
    say(f"full-size {wl.name} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} shards={wl.shards}")
    d = gen.decode_inputs(wl, dev)
    shards = [ca.dcp.build_shard_cache(d["k_seq"], d["v_seq"], d["offsets"], d["ctx"], r, wl.shards,
                                       wl.interleave, wl.block_size, d["block_rand"]) for r in range(wl.shards)]
    run = ca.dcp.DcpDecode(d["q"], shards)
    o, lse = run.run()
    torch.cuda.synchronize()
    ctx = d["ctx"]
    picks = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 13})
    scale = oracle.default_scale(wl.D)
    for b in picks:
        s0, s1 = int(d["offsets"][b]), int(d["offsets"][b + 1])
        kb, vb = d["k_seq"][s0:s1].cpu(), d["v_seq"][s0:s1].cpu()
        for r in range(wl.shards):
            po, pl = oracle.decode_shard_partial(d["q"][b].cpu(), kb, vb, r, wl.interleave, wl.shards, scale)
            check(f"seq {b} (ctx {s1 - s0}) shard {r}", run.o_parts[r, b], run.lse_parts[r, b], po, pl)
        fo, fl = oracle.decode_full(d["q"][b].cpu(), kb, vb, scale)
        check(f"seq {b} (ctx {s1 - s0}) merged", o[b], lse[b], fo, fl)
    del d, shards, run
    torch.cuda.empty_cache()


def test_dcp_decode_active_fullsize(ca):
    """The decode leg with a current token, as timed: N resident tokens per sequence on the
    shards plus the new token at position N on its owner shard; the merged result against
    attention over all N + 1 tokens."""
    wl = workloads.workload("dcp_decode_gqa")
    dev = torch.device("cuda:0")
    say(f"full-size {wl.name} with current token")
    d = gen.decode_inputs(wl, dev)
    shards = [ca.dcp.build_shard_cache(d["k_seq"], d["v_seq"], d["offsets"], d["ctx"], r, wl.shards,
                                       wl.interleave, wl.block_size, d["block_rand"]) for r in range(wl.shards)]
    run = ca.dcp.DcpDecode(d["q"], shards)
    prior = torch.tensor([int(n) for n in d["ctx"]], dtype=torch.int32, device=dev)
    k_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 21, dev, torch.bfloat16)
    v_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 22, dev, torch.bfloat16)
    o, lse = run.run_active(prior, k_cur, v_cur, wl.interleave)
    torch.cuda.synchronize()
    ctx = d["ctx"]
    scale = oracle.default_scale(wl.D)
    for b in sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 5}):
        s0, s1 = int(d["offsets"][b]), int(d["offsets"][b + 1])
        kb = torch.cat([d["k_seq"][s0:s1], k_cur[b:b + 1]]).cpu()
        vb = torch.cat([d["v_seq"][s0:s1], v_cur[b:b + 1]]).cpu()
        fo, fl = oracle.decode_full(d["q"][b].cpu(), kb, vb, scale)
        check(f"seq {b} (ctx {s1 - s0} + current) merged", o[b], lse[b], fo, fl)
    del d, shards, run
    torch.cuda.empty_cache()


def test_dcp_prefill_fullsize(ca):
    """The prefill leg as timed: 8192 new tokens after 65536 prior ones, 32 query heads over 8
    KV heads, DCP 2 interleaving blocks of 16. Sampled chunk rows against attention over the
    prior tokens and the chunk's tokens up to the row."""
    S, P, Hq, Hkv, D, W, I = 8192, 65536, 32, 8, 128, 2, 16
    dev = torch.device("cuda:0")
    say(f"full-size dcp prefill S={S} after {P}")
    q = gen.normal((1, S, Hq, D), 901, dev, torch.bfloat16)
    k_all = gen.normal((P + S, Hkv, D), 902, dev, torch.bfloat16)
    v_all = gen.normal((P + S, Hkv, D), 903, dev, torch.bfloat16)
    caches = [ca.dcp.build_shard_cache(k_all, v_all, np.array([0, P]), np.array([P]), r, W, I, 16) for r in range(W)]
    run = ca.dcp.DcpPrefill(q, k_all[P:].unsqueeze(0), v_all[P:].unsqueeze(0), caches, P, I)
    o, lse = run.run()
    torch.cuda.synchronize()
    scale = oracle.default_scale(D)
    kh_all = oracle.to_f64(k_all.cpu())
    vh_all = oracle.to_f64(v_all.cpu())
    for h in (0, 13, 31):
        rows = _rows(S, 31 * h)
        hk = h // (Hq // Hkv)
        qh = oracle.to_f64(q[0, rows, h].cpu())
        allowed = np.arange(P + S)[None, :] <= (P + rows)[:, None]
        ro, rl = oracle.attention(qh, kh_all[:, hk], vh_all[:, hk], scale, allowed)
        check(f"prefill head {h} ({len(rows)} rows)", o[h, rows], lse[h, rows], ro, rl)
    del q, k_all, v_all, caches, run
    torch.cuda.empty_cache()
