"""Ordering of the ring's K/V hops against the steps that read them.

The ring pass rotates its receive buffers (kernel reference page, Implementation, "The ring
loop": the hop of a later chunk is launched while the current one is computed, into one of
kv_prefetch_depth + 1 buffers). Parity under natural timing cannot show that every step
waits for its chunk and that no hop overwrites a buffer a running step still reads: the
copies usually finish early anyway. Here every receive buffer, partial and accumulator is
filled with NaN before each pass, and a bounded spin (torch.cuda._sleep) is queued ahead of
every hop, on the stream that carries it, and ahead of steps on the second compute stream,
so a missing wait makes a step read NaN or a half-written chunk. Two passes run back to
back, each poisoned, and both must match the fp64 oracle."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check, say
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# about 0.2-0.5 ms of spinning at the shader clock: longer than one small step
SPIN_CYCLES = 1_000_000


@pytest.fixture(scope="module")
def ca():
    import context_attention_lse_amd as ca
    ca._lib.load()
    torch.cuda.set_device(torch.device("cuda:0"))
    return ca


def _spin():
    torch.cuda._sleep(SPIN_CYCLES)


def _delayed(monkeypatch, ca, hop_steps_too):
    """Wraps the library calls the ring driver makes: every chunk copy starts after a spin on
    its stream; with hop_steps_too, so does every step call that carries a hop and every
    step on a stream other than the calling one."""
    api = ca.api
    real_copy = api.kv_chunk_copy
    real_step = api.ring_attn_step
    real_cm = api.ring_attn_const_max_step
    main = torch.cuda.current_stream()
    seen = {"copies": 0, "steps": 0}

    def copy(*a, **kw):
        _spin()
        seen["copies"] += 1
        return real_copy(*a, **kw)

    def wrap(real):
        def step(*a, **kw):
            if hop_steps_too and (kw.get("hop") is not None or torch.cuda.current_stream() != main):
                _spin()
            seen["steps"] += 1
            return real(*a, **kw)
        return step

    monkeypatch.setattr(api, "kv_chunk_copy", copy)
    monkeypatch.setattr(api, "ring_attn_step", wrap(real_step))
    monkeypatch.setattr(api, "ring_attn_const_max_step", wrap(real_cm))
    return seen


def _poison(rp):
    nan = float("nan")
    for b in rp.kbuf + rp.vbuf:
        b.fill_(nan)
    for name in ("o_parts", "lse_parts", "acc", "out", "lse"):
        t = getattr(rp, name, None)
        if t is not None:
            t.fill_(nan)


CASES = [
    # (variant, layout, causal, ring keywords)
    ("online", "contiguous", False, {}),                                        # copy stream, 2 compute streams
    ("online", "contiguous", False, {"prefetch_depth": 3}),
    ("online", "contiguous", False, {"split": True, "compute_streams": 2}),
    ("online", "striped", True, {}),
    ("online", "contiguous", True, {}),                                         # empty steps
    ("constmax", "contiguous", False, {}),
    ("online", "contiguous", False, {"split": True, "compute_streams": 2, "fused_hops": True}),
    ("online", "striped", True, {"fused_hops": True}),
    ("constmax", "contiguous", False, {"fused_hops": True}),
    ("online", "contiguous", False, {"fold": True, "compute_streams": 2}),
    ("online", "contiguous", False, {"fold": True, "compute_streams": 2, "fused_hops": True}),
    ("online", "striped", True, {"fold": True, "fused_hops": True}),
]


@pytest.mark.parametrize("variant,layout,causal,kw", CASES)
def test_ring_with_delayed_hops_and_poisoned_buffers(ca, monkeypatch, variant, layout, causal, kw):
    wl = workloads.workload("wan22_cp8_online").scaled(S=8 * 520, H=2)
    dev = torch.device("cuda:0")
    say(f"ordering variant={variant} layout={layout} causal={causal} {kw} S={wl.S} cp={wl.cp}")
    t = gen.ring_inputs(wl, dev)
    rank = 3
    q = ca.ring.shard(t["q"], wl.cp, rank, layout)
    kp = ca.ring.chunk_pool(t["k"], wl.cp, layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, layout)
    rp = ca.ring.RingPass(q, kp, vp, rank, layout=layout, causal=causal, variant=variant, **kw)
    seen = _delayed(monkeypatch, ca, hop_steps_too=bool(kw.get("fused_hops")) or "compute_streams" in kw)
    tok = (oracle.contiguous_tokens if layout == "contiguous" else oracle.striped_tokens)(wl.S, wl.cp, rank)
    allowed = oracle.causal_allowed(tok, np.arange(wl.S)) if causal else None
    ro, rl = oracle.attention_heads(t["q"][:, tok], t["k"], t["v"], oracle.default_scale(wl.D), allowed=allowed)
    for p in range(2):
        _poison(rp)
        o, lse = rp.run()
        out = o.clone()
        ls = lse.clone()
        torch.cuda.synchronize()
        check(f"pass {p}", out, ls, ro, rl)
    assert seen["copies"] + seen["steps"] > 0
    say(f"  delayed calls: {seen}")
