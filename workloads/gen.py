"""Seeded random tensors for the workloads in ``workloads.configs``.

Conventions:
- every tensor is drawn in fp32 by ``torch.randn`` from its own ``torch.Generator``
  (seed = 1000 * workload seed + a per-tensor offset), in row chunks of a fixed
  size so that the draw does not depend on how much memory is free, then rounded
  to the workload dtype by torch's round-to-nearest-even cast;
- the same call on the same device type gives the same bits; values differ
  between CPU and GPU generators, which is fine because the oracle always reads
  back the very tensor the GPU consumed;
- integer draws (context lengths, block shuffles) use a CPU generator so they are
  identical everywhere.
"""

import math

import numpy as np
import torch

_DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}
_CHUNK_ROWS = 8192


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def _generator(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev.type if dev.type == "cpu" else dev)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0,1) tensor of ``shape``; drawn as [shape[0]*..., last] row chunks."""
    shape = tuple(int(s) for s in shape)
    cols = shape[-1] if shape else 1
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    out = torch.empty((rows, cols), dtype=dtype, device=device)
    g = _generator(seed, device)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        out[r0:r1] = torch.randn((r1 - r0, cols), generator=g, device=device,
                                 dtype=torch.float32).to(dtype)
    return out.reshape(shape)


def rms_normed_heads(tokens: int, heads_total: int, heads_keep: int, head_dim: int,
                     seed: int, device="cpu", dtype=torch.bfloat16, eps: float = 1e-6):
    """Per-token RMS normalisation across all ``heads_total * head_dim`` features
    (learned gain 1), then the first ``heads_keep`` heads. Shape [tokens, heads_keep, head_dim].

    This mimics the statistics of a model that normalises Q and K across its whole
    hidden size before splitting into heads, so individual heads' norms float while
    the total energy per token is pinned.
    """
    hid = heads_total * head_dim
    out = torch.empty((tokens, heads_keep, head_dim), dtype=dtype, device=device)
    g = _generator(seed, device)
    for t0 in range(0, tokens, _CHUNK_ROWS):
        t1 = min(tokens, t0 + _CHUNK_ROWS)
        x = torch.randn((t1 - t0, hid), generator=g, device=device, dtype=torch.float32)
        x = x * torch.rsqrt(x.pow(2).mean(dim=1, keepdim=True) + eps)
        out[t0:t1] = x[:, : heads_keep * head_dim].reshape(t1 - t0, heads_keep, head_dim).to(dtype)
    return out


def ring_inputs(wl, device="cpu", S=None):
    """Global Q, K, V as [B, S, H, D] tensors in the workload dtype.

    ``S`` overrides the workload's global length (small parity cases)."""
    S = int(wl.S if S is None else S)
    dt = torch_dtype(wl.dtype)
    out = {}
    for i, name in enumerate(("q", "k", "v")):
        seed = 1000 * wl.seed + 1 + i
        if wl.qk_norm and name in ("q", "k"):
            parts = [rms_normed_heads(S, wl.H_total, wl.H, wl.D, seed + 97 * b, device, dt)
                     for b in range(wl.B)]
            t = torch.stack(parts, 0)
        else:
            t = normal((wl.B, S, wl.H, wl.D), seed, device, dt)
        out[name] = t
    return out


def context_lengths(wl) -> np.ndarray:
    if wl.ctx_override is not None:
        return np.asarray(wl.ctx_override, dtype=np.int64)
    g = torch.Generator().manual_seed(1000 * wl.seed + 11)
    return torch.randint(wl.ctx_min, wl.ctx_max + 1, (wl.B,), generator=g).numpy().astype(np.int64)


def decode_inputs(wl, device="cpu"):
    """Decode inputs.

    Returns a dict with
      q        [B, Hq, D]           one query token per sequence
      ctx      [B] int64 (numpy)    context length of each sequence
      offsets  [B+1] int64 (numpy)  start of each sequence in k_seq / v_seq
      k_seq    [sum(ctx), Hkv, D]   keys of every sequence, in token order
      v_seq    [sum(ctx), Hkv, D]   values, same layout
      block_rand  float64 numpy     uniform draws a cache allocator may use to
                                    shuffle physical block ids (one per possible block)
    """
    dt = torch_dtype(wl.dtype)
    ctx = context_lengths(wl)
    offsets = np.zeros(wl.B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(ctx)
    total = int(offsets[-1])
    q = normal((wl.B, wl.Hq, wl.D), 1000 * wl.seed + 1, device, dt)
    k_seq = normal((total, wl.Hkv, wl.D), 1000 * wl.seed + 2, device, dt)
    v_seq = normal((total, wl.Hkv, wl.D), 1000 * wl.seed + 3, device, dt)
    n_rand = int(sum(math.ceil(int(c) / wl.block_size) + wl.shards for c in ctx))
    g = torch.Generator().manual_seed(1000 * wl.seed + 13)
    block_rand = torch.rand((n_rand,), generator=g, dtype=torch.float64).numpy()
    return {"q": q, "ctx": ctx, "offsets": offsets, "k_seq": k_seq, "v_seq": v_seq,
            "block_rand": block_rand}


def sample_rows(n_rows: int, n_sample: int, seed: int, include=()) -> np.ndarray:
    """Sorted unique row indices: ``include`` plus ``n_sample`` seeded uniform picks."""
    rng = np.random.default_rng(seed)
    picks = rng.integers(0, n_rows, size=max(0, int(n_sample)))
    extra = [int(i) for i in include if 0 <= int(i) < n_rows]
    return np.unique(np.concatenate([picks, np.asarray(extra, dtype=np.int64)])).astype(np.int64)
