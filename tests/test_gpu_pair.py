"""ring_attn_step_pair: two ring steps in one launch equal attention over both chunks' keys
(the fp64 oracle), and the hops the launch carries arrive byte for byte; the ring pass that
pairs its steps (RingPass(pair_steps=True)) matches the oracle with every receive buffer
poisoned before each pass, eagerly and replayed as a HIP graph."""

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
    torch.cuda.set_device(torch.device("cuda:0"))
    return ca


def _chunk(B, S, H, seed):
    dev = torch.device("cuda:0")
    return [gen.normal((B, S, H, 128), seed + i, dev, torch.bfloat16) for i in range(2)]


def _hop():
    dev = torch.device("cuda:0")
    src = [torch.randint(-2**31, 2**31 - 1, (1_000_003 * 4,), dtype=torch.int32, device=dev) for _ in range(2)]
    return (torch.zeros_like(src[0]), torch.zeros_like(src[1]), src[0], src[1])


# (B, H, Sq, Sk1, Sk2, split, fold, heads checked against the oracle): the Wan2.2 share (160
# query tiles: the hops ride in the launch's free CUs); a ragged second chunk folded into a
# prior; a key-split workspace; an empty first chunk; an empty second chunk
CASES = [(1, 10, 4096, 4096, 4096, False, False, (0, 9)), (2, 2, 300, 256, 200, False, True, None),
         (1, 3, 1000, 512, 333, True, False, None), (1, 2, 257, 0, 100, False, False, None),
         (1, 2, 129, 96, 0, False, True, None)]


@pytest.mark.parametrize("B,H,Sq,Sk1,Sk2,split,fold,heads", CASES)
def test_step_pair_matches_oracle_and_carries_hops(ca, B, H, Sq, Sk1, Sk2, split, fold, heads):
    say(f"step pair B={B} H={H} Sq={Sq} Sk1={Sk1} Sk2={Sk2} split={split} fold={fold}")
    dev = torch.device("cuda:0")
    q = gen.normal((B, Sq, H, 128), 800, dev, torch.bfloat16)
    k0, v0 = _chunk(B, 77, H, 810)
    k1, v1 = _chunk(B, Sk1, H, 820)
    k2, v2 = _chunk(B, Sk2, H, 830)
    # the second chunk with the first chunk's strides (one kv_strides for both)
    if Sk2 and Sk1:
        k2 = torch.empty_strided(k2.shape, k1.stride(), dtype=k2.dtype, device=dev).copy_(k2)
        v2 = torch.empty_strided(v2.shape, v1.stride(), dtype=v2.dtype, device=dev).copy_(v2)
    out = lse = None
    if fold:
        out, lse = ca.api.ring_attn_step(q, k0, v0)
    ws = None
    if split:
        n = ca.api.ring_attn_workspace_size(torch.bfloat16, B, H, Sq, Sk1 + Sk2, 128)
        ws = torch.zeros(n, dtype=torch.uint8, device=dev) if n else None
    hops = [_hop(), _hop()]
    o, l = ca.api.ring_attn_step_pair(q, k1, v1, k2, v2, out=out, lse=lse, fold=fold, workspace=ws, hops=hops)
    torch.cuda.synchronize()
    for dk, dv, sk, sv in hops:
        assert torch.equal(dk, sk) and torch.equal(dv, sv), "hop bytes differ"
    ks = ([k0] if fold else []) + [k1, k2]
    vs = ([v0] if fold else []) + [v1, v2]
    k, v = torch.cat(ks, 1), torch.cat(vs, 1)
    scale = oracle.default_scale(128)
    hh = range(H) if heads is None else heads
    for h in hh:
        for b in range(B):
            ro, rl = oracle.attention(q[b, :, h], k[b, :, h], v[b, :, h], scale)
            check(f"pair b={b} h={h}", o[b, h], l[b, h], ro, rl, quiet=True)
    # the same chunks as separate steps, each after the first folded: the same result up to
    # summation order
    parts = ([(k0, v0)] if fold else []) + [(kk, vv) for kk, vv in ((k1, v1), (k2, v2)) if kk.shape[1]]
    o2 = l2 = None
    for i, (kk, vv) in enumerate(parts):
        o2, l2 = ca.api.ring_attn_step(q, kk, vv, out=o2, lse=l2, fold=i > 0)
    torch.cuda.synchronize()
    assert float((o - o2).abs().max()) < 2e-3 and float((l - l2).abs().max()) < 1e-4


def test_step_pair_rejects_unsupported(ca):
    dev = torch.device("cuda:0")
    q = gen.normal((1, 64, 2, 128), 840, dev, torch.bfloat16)
    k1, v1 = _chunk(1, 100, 2, 850)   # 100 keys: not a multiple of 32
    k2, v2 = _chunk(1, 100, 2, 860)
    with pytest.raises(ca.CtxAttnError, match="multiple of 32"):
        ca.api.ring_attn_step_pair(q, k1, v1, k2, v2)
    q64 = gen.normal((1, 64, 2, 64), 870, dev, torch.bfloat16)
    k3 = gen.normal((1, 64, 2, 64), 871, dev, torch.bfloat16)
    with pytest.raises(ca.CtxAttnError, match="head_dim 128"):
        ca.api.ring_attn_step_pair(q64, k3, k3, k3, k3)


def _poison(rp):
    for t in rp.kbuf + rp.vbuf:
        t.fill_(float("nan"))


@pytest.mark.parametrize("cp,rank", [(8, 0), (8, 5), (5, 2), (2, 1)])
def test_ring_pair_steps_match_oracle(ca, cp, rank):
    """Paired steps over the ring (an odd cp ends in a single step), receive buffers
    NaN-filled before each pass: a hop that lands late or in the wrong buffer shows."""
    wl = workloads.workload("wan22_cp8_online").scaled(S=cp * 256, cp=cp, H=2)
    say(f"ring pair cp={cp} rank={rank}")
    dev = torch.device("cuda:0")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], cp, rank, wl.layout)
    kp = ca.ring.chunk_pool(t["k"], cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], cp, wl.layout)
    rp = ca.ring.RingPass(q, kp, vp, rank, layout=wl.layout, fold=True, fused_hops=True, pair_steps=True)
    rows = oracle.contiguous_tokens(wl.S, cp, rank)
    ro, rl = oracle.attention_heads(t["q"][:, rows], t["k"], t["v"], oracle.default_scale(wl.D))
    for rep in range(2):
        _poison(rp)
        o, l = rp.run()
        torch.cuda.synchronize()
        check(f"pass {rep}", o, l, ro, rl)
    # replayed as a HIP graph, with eager passes between the replays
    g = rp.capture()
    for rep in range(3):
        _poison(rp)
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}", rp.out, rp.lse, ro, rl)
        _poison(rp)
        rp.run()
        torch.cuda.synchronize()
        check(f"eager after replay {rep}", rp.out, rp.lse, ro, rl)


def test_ring_pair_steps_rejects_unsupported(ca):
    wl = workloads.workload("wan22_cp8_online").scaled(S=8 * 100, H=2)
    dev = torch.device("cuda:0")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], 8, 0, wl.layout)
    kp = ca.ring.chunk_pool(t["k"], 8, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], 8, wl.layout)
    with pytest.raises(ValueError, match="multiple of 32"):
        ca.ring.RingPass(q, kp, vp, 0, fold=True, fused_hops=True, pair_steps=True)
    with pytest.raises(ValueError, match="fused_hops"):
        ca.ring.RingPass(q, kp, vp, 0, fold=True, pair_steps=True)
