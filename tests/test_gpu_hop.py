"""ring_attn_step_hop: the step's outputs are those of ring_attn_step (same kernels, same
arithmetic), and the hop's destinations hold the sources' bytes, whether the hop runs in
the step's launch (CUs the step leaves free) or as a copy ahead of it; and the ring pass
that carries every hop in its steps matches the fp64 oracle."""

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
    torch.cuda.set_device(torch.device("cuda:0"))
    return ca


def _qkv(B, Sq, Sk, H, seed, dtype="bf16"):
    dev = torch.device("cuda:0")
    dt = gen.torch_dtype(dtype)
    q = gen.normal((B, Sq, H, 128 if dtype == "bf16" else 64), seed, dev, dt)
    k = gen.normal((B, Sk, H, q.shape[3]), seed + 1, dev, dt)
    v = gen.normal((B, Sk, H, q.shape[3]), seed + 2, dev, dt)
    return q, k, v


# (B, H, Sq, Sk, mask, split, dtype): 160 query tiles on a key split (240 ranges, 16 CUs
# free: the hop runs in the launch); 16 tiles on a key split (256 ranges, none free: a copy
# ahead); 4 tiles unsplit (most CUs free); causal and fp32 (copy ahead); no rows (hop only)
CASES = [(1, 10, 4096, 4096, "none", True, "bf16"), (1, 2, 2048, 4096, "none", True, "bf16"),
         (2, 2, 512, 700, "none", False, "bf16"), (1, 3, 1000, 1000, "causal_incl", True, "bf16"),
         (1, 2, 300, 200, "none", False, "fp32"), (1, 2, 0, 64, "none", False, "bf16")]


@pytest.mark.parametrize("B,H,Sq,Sk,mask,split,dtype", CASES)
def test_step_hop_matches_step_and_copies(ca, B, H, Sq, Sk, mask, split, dtype):
    say(f"step_hop B={B} H={H} Sq={Sq} Sk={Sk} mask={mask} split={split} dtype={dtype}")
    q, k, v = _qkv(B, Sq, Sk, H, 700, dtype)
    ws = ca.api.step_workspace(q, k, mask) if split else None
    o0, l0 = ca.api.ring_attn_step(q, k, v, mask=mask, workspace=ws)
    # a chunk-sized hop with recognisable bytes, not a multiple of the copy stride
    src_k = torch.randint(-2**31, 2**31 - 1, (1_000_003 * 4,), dtype=torch.int32, device=q.device)
    src_v = torch.randint(-2**31, 2**31 - 1, (1_000_003 * 4,), dtype=torch.int32, device=q.device)
    dst_k = torch.zeros_like(src_k)
    dst_v = torch.zeros_like(src_v)
    o1, l1 = ca.api.ring_attn_step(q, k, v, mask=mask, workspace=ws, hop=(dst_k, dst_v, src_k, src_v))
    torch.cuda.synchronize()
    assert torch.equal(dst_k, src_k) and torch.equal(dst_v, src_v), "hop bytes differ"
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "step outputs differ with the hop"


@pytest.mark.parametrize("B,H,Sq,Sk,mask,split", [(1, 10, 4096, 4096, "none", False), (2, 2, 512, 700, "none", False),
                                                  (1, 3, 1000, 1000, "causal_strict", True)])
def test_step_fold_hop_matches_step_fold_and_copies(ca, B, H, Sq, Sk, mask, split):
    """ring_attn_step_fold_hop: the fold of ring_attn_step_fold, bit for bit, and the hop's bytes."""
    say(f"step_fold_hop B={B} H={H} Sq={Sq} Sk={Sk} mask={mask} split={split}")
    q, k1, v1 = _qkv(B, Sq, Sk, H, 720)
    _, k2, v2 = _qkv(B, Sq, Sk, H, 730)
    ws = ca.api.step_workspace(q, k2, mask) if split else None
    o0, l0 = ca.api.ring_attn_step(q, k1, v1, mask=mask)
    o1, l1 = o0.clone(), l0.clone()
    ca.api.ring_attn_step(q, k2, v2, mask=mask, out=o0, lse=l0, fold=True, workspace=ws)
    src_k = torch.randint(-2**31, 2**31 - 1, (1_000_003 * 4,), dtype=torch.int32, device=q.device)
    src_v = torch.randint(-2**31, 2**31 - 1, (1_000_003 * 4,), dtype=torch.int32, device=q.device)
    dst_k = torch.zeros_like(src_k)
    dst_v = torch.zeros_like(src_v)
    ca.api.ring_attn_step(q, k2, v2, mask=mask, out=o1, lse=l1, fold=True, workspace=ws,
                          hop=(dst_k, dst_v, src_k, src_v))
    torch.cuda.synchronize()
    assert torch.equal(dst_k, src_k) and torch.equal(dst_v, src_v), "hop bytes differ"
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "fold outputs differ with the hop"


def test_step_hop_rejects_bad_buffers(ca):
    q, k, v = _qkv(1, 64, 64, 1, 710)
    a = torch.zeros(64, dtype=torch.uint8, device=q.device)
    with pytest.raises(ValueError):
        ca.api.ring_attn_step(q, k, v, hop=(a, a[:32], a, a))
    # 24 bytes: not a multiple of 16 (checked by the library)
    b = torch.zeros(24, dtype=torch.uint8, device=q.device)
    with pytest.raises(ca._lib.CtxAttnError) as e:
        ca.api.ring_attn_step(q, k, v, hop=(b, b.clone(), b.clone(), b.clone()))
    assert e.value.status == ca._lib.CA_ERR_SHAPE


@pytest.mark.parametrize("wl_name,S,ranks,streams,H,layout,kw", [
    ("wan22_cp8_online", 8 * 328, (0, 5), 2, None, None, {"split": True}),
    ("wan22_cp8_online", 8 * 328, (3,), 1, None, None, {"split": True}),
    ("striped_causal_128k", 8 * 200, (0, 7), 2, 2, None, {"split": True}),
    # contiguous causal: rank 0 sees only its own chunk, so every later step is empty and
    # its hop moves as a plain copy on that step's stream
    ("striped_causal_128k", 8 * 200, (0, 5), 2, 2, "contiguous", {"split": True}),
    # steps folding into one running partial per compute stream, 2-way merge at the end
    ("wan22_cp8_online", 8 * 328, (0, 5), 2, None, None, {"fold": True}),
    ("wan22_cp8_online", 8 * 328, (3,), 1, None, None, {"fold": True}),
    ("striped_causal_128k", 8 * 200, (0, 7), 2, 2, None, {"fold": True}),
    ("striped_causal_128k", 8 * 200, (0, 5), 2, 2, "contiguous", {"fold": True})])
def test_ring_fused_hops_matches_oracle(ca, wl_name, S, ranks, streams, H, layout, kw):
    dev = torch.device("cuda:0")
    wl = workloads.workload(wl_name).scaled(S=S, **({"H": H} if H else {}))
    if layout is not None:
        wl = wl.scaled(layout=layout)
    t = gen.ring_inputs(wl, dev)
    scale = oracle.default_scale(wl.D)
    for r in ranks:
        say(f"ring fused hops {wl.name} S={S} rank={r} streams={streams} {kw}")
        o, l = ca.ring.ring_attention(t["q"], t["k"], t["v"], wl.cp, r, layout=wl.layout, causal=wl.causal,
                                      compute_streams=streams, fused_hops=True, **kw)
        torch.cuda.synchronize()
        rows = (oracle.contiguous_tokens if wl.layout == "contiguous" else oracle.striped_tokens)(S, wl.cp, r)
        allowed = oracle.causal_allowed(rows, np.arange(S)) if wl.causal else None
        ro, rl = oracle.attention_heads(t["q"][:, rows], t["k"], t["v"], scale, allowed=allowed)
        check(f"rank {r}", o, l, ro, rl)


@pytest.mark.parametrize("phase", [1, 0, 2, 3])
def test_const_max_step_hop_matches_step(ca, phase):
    # 720p-like share scaled down: 4 heads x 1000 rows unsplit (CUs free: in the launch)
    say(f"const-max step_hop phase={phase}")
    q, k, v = _qkv(1, 1000, 900, 4, 720)
    c = ca.api.const_max_bound(q, ca.api.key_sqnorm_max(k))
    n = ca.api.const_max_acc_size(1, 4, 1000, 128)
    acc0 = gen.normal((n,), 721, q.device, torch.float32).abs()
    acc1 = acc0.clone()
    r0 = ca.api.ring_attn_const_max_step(q, k, v, c, acc0, phase)
    src_k = torch.randint(-2**31, 2**31 - 1, (300_001 * 4,), dtype=torch.int32, device=q.device)
    src_v = torch.randint(-2**31, 2**31 - 1, (300_001 * 4,), dtype=torch.int32, device=q.device)
    dst_k, dst_v = torch.zeros_like(src_k), torch.zeros_like(src_v)
    r1 = ca.api.ring_attn_const_max_step(q, k, v, c, acc1, phase, hop=(dst_k, dst_v, src_k, src_v))
    torch.cuda.synchronize()
    assert torch.equal(dst_k, src_k) and torch.equal(dst_v, src_v), "hop bytes differ"
    if phase & 2:
        assert torch.equal(r0[0], r1[0]) and torch.equal(r0[1], r1[1])
    if phase != 3:
        assert torch.equal(acc0, acc1)


def test_ring_const_max_fused_hops_matches_oracle(ca):
    dev = torch.device("cuda:0")
    wl = workloads.workload("wan22_720p_constmax").scaled(S=8 * 300, H=4)
    t = gen.ring_inputs(wl, dev)
    scale = oracle.default_scale(wl.D)
    rows = oracle.contiguous_tokens(wl.S, wl.cp, 0)
    say(f"const-max ring fused hops {wl.name} S={wl.S}")
    o, l = ca.ring.ring_attention(t["q"], t["k"], t["v"], wl.cp, 0, variant="constmax", fused_hops=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_heads(t["q"][:, rows], t["k"], t["v"], scale)
    check("rank 0", o, l, ro, rl)
