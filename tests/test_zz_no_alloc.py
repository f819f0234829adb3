"""dcp_decode_partial_noalloc: the decode entry point that allocates nothing (its split partials
live in the library's fixed per-GPU scratch) gives the same outputs as dcp_decode_partial with a
caller workspace, on two calls in a row (the second smaller), through the C ABI; sizes over the
scratch limit are refused before anything is launched."""

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


def _case(ca, B, Hq, Hkv, ctx, seed):
    wl = workloads.workload("dcp_decode_gqa").scaled(B=B, Hq=Hq, Hkv=Hkv, ctx_override=tuple(ctx), seed=seed)
    d = gen.decode_inputs(wl, torch.device("cuda:0"))
    shards = [ca.dcp.build_shard_cache(d["k_seq"], d["v_seq"], d["offsets"], d["ctx"], r, 2, 16, 16, d["block_rand"])
              for r in range(2)]
    return wl, d, shards


@pytest.mark.parametrize("order", ["large_then_small"])
def test_decode_noalloc_matches_workspace_entry_point(ca, order):
    cases = [(6, 64, 8, (70001, 1, 16, 1023, 33000, 5000), 41), (2, 16, 2, (300, 2100), 42)]
    for i, (B, Hq, Hkv, ctx, seed) in enumerate(cases):
        say(f"noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} ctx={ctx}")
        wl, d, shards = _case(ca, B, Hq, Hkv, ctx, seed)
        scale = oracle.default_scale(wl.D)
        for r, sc in enumerate(shards):
            o_ws, l_ws = ca.dcp_decode_partial(d["q"], sc.k_pool, sc.v_pool, sc.block_table, sc.local_lens)
            o_na = torch.full_like(o_ws, float("nan"))
            l_na = torch.full_like(l_ws, float("nan"))
            ca.dcp_decode_partial_noalloc(d["q"], sc.k_pool, sc.v_pool, sc.block_table, sc.local_lens,
                                          out=o_na, lse=l_na)
            torch.cuda.synchronize()
            # the same kernels and arithmetic on the same inputs: identical bits
            assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), f"call {i} shard {r}: outputs differ"
            for b in range(B):
                s0, s1 = int(d["offsets"][b]), int(d["offsets"][b + 1])
                po, pl = oracle.decode_shard_partial(d["q"][b], d["k_seq"][s0:s1], d["v_seq"][s0:s1], r, 16, 2, scale)
                check(f"call {i} shard {r} seq {b} (ctx {s1 - s0})", o_na[b], l_na[b], po, pl, quiet=True)
        say(f"  call {i}: identical to dcp_decode_partial on both shards, within the bar of the oracle")


def test_decode_noalloc_refuses_sizes_over_the_scratch(ca):
    # 64 sequences x 64 heads x 87 splits x 129 x 4 bytes = 184 MB > 80 MiB of scratch
    dev = torch.device("cuda:0")
    q = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device=dev)
    kp = torch.zeros((1, 8, 16, 128), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros((1, 8, 128, 16), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((64, 8192), dtype=torch.int32, device=dev)
    lens = torch.zeros((64,), dtype=torch.int32, device=dev)
    with pytest.raises(ca.CtxAttnError, match="scratch"):
        ca.dcp_decode_partial_noalloc(q, kp, vp, bt, lens)
    torch.cuda.synchronize()
