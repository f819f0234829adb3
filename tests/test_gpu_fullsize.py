"""HIP path vs the fp64 oracle at the workloads' full sizes, in the launch configuration the
benchmark times (RingPass / DcpDecode with the benchmark's options).

Coverage, element by element against the oracle (the kernel reference page, "Adapting this
kernel": validate against exact attention computed on the CPU):
- Wan2.2 share (S = 32768, cp = 8, 10 heads): every row of every head of the pass;
- 720p const-max (S = 75600, cp = 8, 40 heads): every row of heads 0 and 39, plus sampled
  rows of every other head; the online pass on sampled rows;
- striped causal S = 128k: every row of head 0 of rank 7, sampled rows of every head of
  ranks 0, 3 and 7 (folded steps, as timed), and of four heads of rank 5 (merged partials);
- DCP decode (32 sequences, both shards): every sequence's shard partials and merged
  result, with and without the current token;
- DCP prefill chunk: sampled rows of three heads.
Sampled rows always include the first rows, both sides of the 256-row query-tile edges,
the ragged last tile and the last row."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check, say, to_np
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROW_CHUNK = 1024   # oracle rows per call (bounds the causal mask's memory)


@pytest.fixture(scope="module")
def ca():
    import context_attention_lse_amd as ca
    ca._lib.load()
    torch.cuda.set_device(0)
    return ca


def _rows(n, seed, k=24):
    last_tile = (n - 1) // 256 * 256
    return gen.sample_rows(n, k, seed, include=(0, 1, 255, 256, last_tile - 1, last_tile, n - 2, n - 1))


def _ring_pass(ca, name, variant, rank, contiguous_q, **ring_kw):
    """Runs one rank's ring pass as the benchmark does; returns the inputs (on the GPU),
    the outputs (on the host) and the rank's global token positions."""
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
    o, lse = o.cpu(), lse.cpu()
    del q, kp, vp, rp
    torch.cuda.empty_cache()
    tok = (oracle.contiguous_tokens if wl.layout == "contiguous" else oracle.striped_tokens)(wl.S, wl.cp, rank)
    return wl, t, o, lse, tok


def _check_head(label, wl, t, o, lse, tok, h, rows):
    """Rows ``rows`` of head h against the oracle over the full key range."""
    scale = oracle.default_scale(wl.D)
    kh = oracle.to_f64(t["k"][0, :, h])
    vh = oracle.to_f64(t["v"][0, :, h])
    eo = el = 0.0
    for r0 in range(0, len(rows), ROW_CHUNK):
        rr = rows[r0:r0 + ROW_CHUNK]
        qh = oracle.to_f64(t["q"][0, tok[rr], h])
        allowed = oracle.causal_allowed(tok[rr], np.arange(wl.S)) if wl.causal else None
        ro, rl = oracle.attention(qh, kh, vh, scale, allowed)
        e = check(f"{label} head {h} rows {rr[0]}..{rr[-1]}", o[0, h, rr], lse[0, h, rr], ro, rl, quiet=True)
        eo, el = max(eo, e[0]), max(el, e[1])
    say(f"  {label} head {h} ({len(rows)} rows): max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    return eo, el


def _summary(label, errs):
    eo = max(e[0] for e in errs)
    el = max(e[1] for e in errs)
    say(f"{label}: max|dO|={eo:.3e} max|dLSE|={el:.3e} over {len(errs)} head checks")


def test_wan22_cp8_online_fullsize_every_row(ca):
    # the Wan2.2 share in its timed form: unsplit steps alternating two compute streams (two
    # in flight), each carrying the hop of the chunk two steps ahead and folding into its
    # stream's running partial; every row of every head
    wl, t, o, lse, tok = _ring_pass(ca, "wan22_cp8_online", "online", 0, False, split=False, compute_streams=2,
                                    fused_hops=True, fold=True)
    errs = [_check_head("wan22 online rank 0", wl, t, o, lse, tok, h, np.arange(wl.local_S)) for h in range(wl.H)]
    _summary("wan22_cp8_online every row", errs)


def test_wan22_cp8_online_fullsize_keysplit_every_row(ca):
    # the same pass with key-split steps (240 key ranges per step: every query tile is cut in
    # two segments combined through the workspace); every row of every head
    wl, t, o, lse, tok = _ring_pass(ca, "wan22_cp8_online", "online", 0, False, split=True, compute_streams=2,
                                    fused_hops=True)
    errs = [_check_head("wan22 key-split rank 0", wl, t, o, lse, tok, h, np.arange(wl.local_S)) for h in range(wl.H)]
    _summary("wan22_cp8_online key-split every row", errs)


def test_wan22_cp8_online_fullsize_copy_stream(ca):
    # the same with the hops on a copy stream
    wl, t, o, lse, tok = _ring_pass(ca, "wan22_cp8_online", "online", 3, False, split=True, compute_streams=2)
    errs = [_check_head("wan22 copy stream rank 3", wl, t, o, lse, tok, h, _rows(wl.local_S, 17 * h + 3))
            for h in range(wl.H)]
    _summary("wan22_cp8_online copy stream", errs)


def test_wan22_cp8_online_fullsize_unsplit(ca):
    wl, t, o, lse, tok = _ring_pass(ca, "wan22_cp8_online", "online", 5, False)
    errs = [_check_head("wan22 unsplit rank 5", wl, t, o, lse, tok, h, _rows(wl.local_S, 17 * h + 5))
            for h in (2, 7)]
    _summary("wan22_cp8_online unsplit", errs)


def test_wan22_720p_constmax_fullsize(ca):
    # the timed const-max pass (steps carry their hops): every row of heads 0 and 39, and
    # sampled rows of every other head
    wl, t, o, lse, tok = _ring_pass(ca, "wan22_720p_constmax", "constmax", 0, True, fused_hops=True)
    errs = [_check_head("720p constmax", wl, t, o, lse, tok, h, np.arange(wl.local_S)) for h in (0, wl.H - 1)]
    errs += [_check_head("720p constmax", wl, t, o, lse, tok, h, _rows(wl.local_S, 17 * h)) for h in range(1, wl.H - 1)]
    _summary("wan22_720p_constmax", errs)


def test_wan22_720p_online_fullsize(ca):
    wl, t, o, lse, tok = _ring_pass(ca, "wan22_720p_constmax", "online", 0, True)
    errs = [_check_head("720p online", wl, t, o, lse, tok, h, _rows(wl.local_S, 19 * h)) for h in range(0, wl.H, 3)]
    _summary("wan22_720p online", errs)


def test_wan22_720p_constmax_sinks_fullsize(ca):
    """The sink-robust pass as timed (theta 4): exact attention is the target whether or not
    any key qualifies as a sink."""
    wl, t, o, lse, tok = _ring_pass(ca, "wan22_720p_constmax", "constmax", 0, True, sink_theta=4.0)
    errs = [_check_head("720p sinks", wl, t, o, lse, tok, h, _rows(wl.local_S, 23 * h)) for h in (0, 17, 39)]
    _summary("wan22_720p sink-robust", errs)


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_striped_causal_128k_fullsize(ca, rank):
    # the timed form: one compute stream folding each step into the running partial, hops on
    # a copy stream
    wl, t, o, lse, tok = _ring_pass(ca, "striped_causal_128k", "online", rank, True, fold=True, compute_streams=1)
    errs = []
    if rank == 7:
        errs.append(_check_head(f"striped rank {rank}", wl, t, o, lse, tok, 0, np.arange(wl.local_S)))
    heads = range(1 if rank == 7 else 0, wl.H)
    errs += [_check_head(f"striped rank {rank}", wl, t, o, lse, tok, h, _rows(wl.local_S, 29 * h + rank, k=8))
             for h in heads]
    _summary(f"striped_causal_128k rank {rank}", errs)


def test_striped_causal_128k_fullsize_merged_partials(ca):
    """The same ring with two compute streams and the 8-way merge of the steps' partials."""
    wl, t, o, lse, tok = _ring_pass(ca, "striped_causal_128k", "online", 5, True)
    errs = [_check_head("striped rank 5 merged", wl, t, o, lse, tok, h, _rows(wl.local_S, 37 * h, k=16))
            for h in (0, 9, 18, 31)]
    _summary("striped_causal_128k rank 5, merged partials", errs)


def test_contiguous_causal_128k_fullsize(ca):
    """The contiguous causal contrast the benchmark times: rank 6 (six full chunks, its own
    triangle, one empty step) on sampled rows of four heads."""
    wl, t, o, lse, tok = _ring_pass(ca, "contiguous_causal_128k", "online", 6, True)
    errs = [_check_head("contiguous causal rank 6", wl, t, o, lse, tok, h, _rows(wl.local_S, 31 * h, k=16))
            for h in (0, 11, 22, 31)]
    _summary("contiguous causal 128k rank 6", errs)


# ---------------------------------------------------------------- DCP decode, every sequence

@pytest.fixture(scope="module")
def decode_run(ca):
    """Both shards' partials and the merged result of the timed decode step, with and
    without the current token, copied to the host; the inputs stay on the GPU."""
    wl = workloads.workload("dcp_decode_gqa")
    dev = torch.device("cuda:0")
    say(f"full-size {wl.name} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} shards={wl.shards}")
    d = gen.decode_inputs(wl, dev)
    shards = [ca.dcp.build_shard_cache(d["k_seq"], d["v_seq"], d["offsets"], d["ctx"], r, wl.shards,
                                       wl.interleave, wl.block_size, d["block_rand"]) for r in range(wl.shards)]
    run = ca.dcp.DcpDecode(d["q"], shards)
    o, lse = run.run()
    res = {"o": o.cpu(), "lse": lse.cpu(), "o_parts": run.o_parts.cpu(), "lse_parts": run.lse_parts.cpu()}
    prior = torch.tensor([int(n) for n in d["ctx"]], dtype=torch.int32, device=dev)
    k_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 21, dev, torch.bfloat16)
    v_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 22, dev, torch.bfloat16)
    oa, la = run.run_active(prior, k_cur, v_cur, wl.interleave)
    res.update({"o_act": oa.cpu(), "lse_act": la.cpu(), "k_cur": k_cur.cpu(), "v_cur": v_cur.cpu()})
    torch.cuda.synchronize()
    del shards, run
    torch.cuda.empty_cache()
    res.update({"wl": wl, "d": d})
    yield res
    del res, d
    torch.cuda.empty_cache()


def _decode_group(q_rows, k_tok, v_tok, keep, scale):
    """The query heads of one GQA group against the group's K/V head restricted to the
    tokens ``keep`` selects (all when None): oracle attention, one row per query head."""
    if keep is not None:
        k_tok, v_tok = k_tok[keep], v_tok[keep]
    return oracle.attention(q_rows, k_tok, v_tok, scale)


@pytest.mark.parametrize("part", range(4))
def test_dcp_decode_fullsize_every_sequence(decode_run, part):
    """Sequences 8*part .. 8*part+7: each shard's partial (the tokens the slot mapping deals
    to it), the merged result (attention over all N tokens), and the merged result with the
    current token at position N."""
    wl, d = decode_run["wl"], decode_run["d"]
    G = wl.Hq // wl.Hkv
    scale = oracle.default_scale(wl.D)
    worst = [0.0, 0.0]
    for b in range(8 * part, 8 * part + 8):
        s0, s1 = int(d["offsets"][b]), int(d["offsets"][b + 1])
        N = s1 - s0
        shard = oracle.dcp_shard_of_position(np.arange(N), wl.interleave, wl.shards)
        q_b = oracle.to_f64(d["q"][b])
        for hk in range(wl.Hkv):
            hs = slice(hk * G, (hk + 1) * G)
            k_tok = oracle.to_f64(d["k_seq"][s0:s1, hk])
            v_tok = oracle.to_f64(d["v_seq"][s0:s1, hk])
            checks = []
            for r in range(wl.shards):
                po, pl = _decode_group(q_b[hs], k_tok, v_tok, shard == r, scale)
                checks.append((f"seq {b} kv head {hk} shard {r}", decode_run["o_parts"][r, b, hs],
                               decode_run["lse_parts"][r, b, hs], po, pl))
            fo, fl = _decode_group(q_b[hs], k_tok, v_tok, None, scale)
            checks.append((f"seq {b} kv head {hk} merged", decode_run["o"][b, hs], decode_run["lse"][b, hs], fo, fl))
            k_all = np.concatenate([k_tok, oracle.to_f64(decode_run["k_cur"][b, hk])[None]])
            v_all = np.concatenate([v_tok, oracle.to_f64(decode_run["v_cur"][b, hk])[None]])
            ao, al = _decode_group(q_b[hs], k_all, v_all, None, scale)
            checks.append((f"seq {b} kv head {hk} merged with current token", decode_run["o_act"][b, hs],
                           decode_run["lse_act"][b, hs], ao, al))
            for name, go, gl, ro, rl in checks:
                e = check(name, go, gl, ro, rl, quiet=True)
                worst = [max(worst[0], e[0]), max(worst[1], e[1])]
        say(f"  seq {b} (ctx {N}): checked; running max|dO|={worst[0]:.3e} max|dLSE|={worst[1]:.3e}")
    say(f"dcp_decode_gqa sequences {8 * part}..{8 * part + 7}: max|dO|={worst[0]:.3e} max|dLSE|={worst[1]:.3e}")


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
