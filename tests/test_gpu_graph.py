"""A ring pass captured as a HIP graph (RingPass.capture): every replay, with the program's
own eager passes and synchronisations between replays, gives the eager pass's bits, and the
result matches the fp64 oracle. The Wan2.2 pass's form: unsplit steps on two compute
streams, hops carried by the steps, each stream folding into a running partial."""

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


@pytest.mark.parametrize("kw,causal,layout", [
    ({"split": False, "compute_streams": 2, "fused_hops": True, "fold": True}, False, "contiguous"),
    ({"split": False, "compute_streams": 2, "fused_hops": True}, False, "contiguous"),
    ({"fold": True, "compute_streams": 1}, True, "striped"),
])
def test_ring_pass_graph_replays_match_eager_and_oracle(ca, kw, causal, layout):
    dev = torch.device("cuda:0")
    wl = workloads.workload("wan22_cp8_online").scaled(S=8 * 520, H=3)
    say(f"graph pass {kw} causal={causal} layout={layout} S={wl.S}")
    t = gen.ring_inputs(wl, dev)
    rank = 2
    q = ca.ring.shard(t["q"], wl.cp, rank, layout)
    kp = ca.ring.chunk_pool(t["k"], wl.cp, layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, layout)
    rp = ca.ring.RingPass(q, kp, vp, rank, layout=layout, causal=causal, variant="online", **kw)
    o_ref, l_ref = (x.clone() for x in rp.run())
    torch.cuda.synchronize()
    g = rp.capture()
    for i in range(4):
        rp.out.fill_(float("nan"))
        rp.lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rp.out, o_ref) and torch.equal(rp.lse, l_ref), f"replay {i} differs from the eager pass"
        rp.run()                     # eager work between replays
        torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    tok = (oracle.contiguous_tokens if layout == "contiguous" else oracle.striped_tokens)(wl.S, wl.cp, rank)
    allowed = oracle.causal_allowed(tok, np.arange(wl.S)) if causal else None
    ro, rl = oracle.attention_heads(t["q"][:, tok], t["k"], t["v"], oracle.default_scale(wl.D), allowed=allowed)
    check("graph replay", rp.out, rp.lse, ro, rl)


def test_capture_refuses_two_compute_streams_with_a_copy_stream(ca):
    """That form is run eagerly only: capture() raises before capturing anything."""
    dev = torch.device("cuda:0")
    wl = workloads.workload("wan22_cp8_online").scaled(S=8 * 64, H=1)
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, 0, "contiguous")
    kp = ca.ring.chunk_pool(t["k"], wl.cp, "contiguous")
    vp = ca.ring.chunk_pool(t["v"], wl.cp, "contiguous")
    rp = ca.ring.RingPass(q, kp, vp, 0, variant="online", fold=True, compute_streams=2)
    with pytest.raises(NotImplementedError):
        rp.capture()
