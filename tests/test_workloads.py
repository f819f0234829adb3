"""Seeded input generators (CPU): determinism and the statistics they promise."""

import math

import numpy as np
import torch

import workloads
from workloads import gen


def test_normal_is_deterministic_and_chunk_independent_of_memory():
    a = gen.normal((3, 5000, 2, 8), seed=42)
    b = gen.normal((3, 5000, 2, 8), seed=42)
    c = gen.normal((3, 5000, 2, 8), seed=43)
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert abs(float(a.mean())) < 0.02 and abs(float(a.std()) - 1.0) < 0.02


def test_rms_normed_heads_pins_total_energy_not_per_head():
    x = gen.rms_normed_heads(2048, 40, 40, 128, seed=3, dtype=torch.float32)
    per_token = x.pow(2).mean(dim=(1, 2))
    assert torch.allclose(per_token, torch.ones_like(per_token), atol=1e-4)
    # individual heads float: per-head squared norm ~ chi^2(128), spread bounded by sqrt(D/d)
    head_norm = x.pow(2).sum(-1).sqrt()
    assert float(head_norm.max()) <= math.sqrt(40 * 128) + 1e-3
    assert float(head_norm.std()) > 0.3
    kept = gen.rms_normed_heads(2048, 40, 10, 128, seed=3, dtype=torch.float32)
    assert torch.equal(kept, x[:, :10])


def test_ring_inputs_shapes_and_dtypes():
    wl = workloads.workload("wan22_cp8_online").scaled(S=256)
    t = gen.ring_inputs(wl)
    for name in "qkv":
        assert t[name].shape == (1, 256, 10, 128) and t[name].dtype == torch.bfloat16
    tiny = gen.ring_inputs(workloads.workload("tiny_ring_fp32"))
    assert tiny["q"].dtype == torch.float32 and tiny["q"].shape == (1, 512, 2, 64)


def test_decode_inputs_context_lengths():
    wl = workloads.workload("dcp_decode_gqa")
    ctx = gen.context_lengths(wl)
    assert ctx.shape == (32,) and ctx.min() >= 32768 and ctx.max() <= 131072
    assert np.array_equal(ctx, gen.context_lengths(wl))
    small = wl.scaled(B=3, ctx_override=(5, 40, 17))
    d = gen.decode_inputs(small)
    assert d["k_seq"].shape == (62, 8, 128) and list(d["offsets"]) == [0, 5, 45, 62]
    assert d["block_rand"].shape[0] >= sum(math.ceil(c / 16) for c in (5, 40, 17))


def test_sample_rows():
    r = gen.sample_rows(100, 10, seed=1, include=(0, 99, 500))
    assert r[0] == 0 and r[-1] == 99 and np.all(np.diff(r) > 0)
