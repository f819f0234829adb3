"""The five synthetic workloads, with the shapes the pages' deployments use.

Shapes follow the Wan2.2 A14B DiT (40 heads of 128, hidden 5120) from the
context-parallelism page and the kernel reference page, the long-context decode
case from the DCP page (64 query heads, 8 KV heads, paged blocks of 16 tokens,
interleave 16, two shards), and striped ring attention from the sequence-sharding
survey page. None of the pages' datasets or weights are used; every tensor is a
seeded random draw (see ``workloads.gen``).
"""

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class RingWorkload:
    """One rank's share of ring attention over ``cp`` K/V chunks."""

    name: str
    B: int
    H: int            # heads computed here
    D: int
    S: int            # global sequence length (all ranks)
    cp: int           # ring size
    dtype: str        # "bf16" or "fp32"
    seed: int
    qk_norm: bool     # Q,K RMS-normalised per token across H_total*D (gain 1)
    H_total: int      # heads the RMS norm spans (the model's full head count)
    layout: str       # "contiguous" (rank r owns tokens [r*S/cp, (r+1)*S/cp)) or "striped" (t -> t % cp)
    causal: bool
    ranks: tuple      # which ranks' shares are computed
    variants: tuple   # subset of ("online", "constmax")

    @property
    def local_S(self) -> int:
        return self.S // self.cp

    def scaled(self, **kw) -> "RingWorkload":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeWorkload:
    """Decode of one query token per sequence against a paged KV cache split over shards."""

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    interleave: int
    shards: int
    ctx_min: int
    ctx_max: int
    dtype: str
    seed: int
    ctx_override: Optional[tuple] = None   # explicit context lengths (small tests)

    def scaled(self, **kw) -> "DecodeWorkload":
        return replace(self, **kw)


WORKLOADS = {
    # 0: tiny fp32 ring, small enough for the oracle to run in full in well under a second.
    "tiny_ring_fp32": RingWorkload(
        name="tiny_ring_fp32", B=1, H=2, D=64, S=512, cp=4, dtype="fp32", seed=1,
        qk_norm=False, H_total=2, layout="contiguous", causal=False, ranks=(0,),
        variants=("online", "constmax")),
    # 1: Wan2.2 DiT self-attention, one rank's share under TP=4 (10 of 40 heads), CP=8.
    "wan22_cp8_online": RingWorkload(
        name="wan22_cp8_online", B=1, H=10, D=128, S=32768, cp=8, dtype="bf16", seed=2,
        qk_norm=True, H_total=40, layout="contiguous", causal=False, ranks=(0,),
        variants=("online",)),
    # 2: Wan2.2 720p x 81 frames (21*45*80 = 75600 tokens), all 40 heads, CP=8: local 9450 (ragged tail).
    "wan22_720p_constmax": RingWorkload(
        name="wan22_720p_constmax", B=1, H=40, D=128, S=75600, cp=8, dtype="bf16", seed=3,
        qk_norm=True, H_total=40, layout="contiguous", causal=False, ranks=(0,),
        variants=("constmax", "online")),
    # 3: DCP decode, 32 sequences, GQA 64/8, paged KV (block 16) interleaved over 2 shards.
    "dcp_decode_gqa": DecodeWorkload(
        name="dcp_decode_gqa", B=32, Hq=64, Hkv=8, D=128, block_size=16, interleave=16,
        shards=2, ctx_min=32768, ctx_max=131072, dtype="bf16", seed=4),
    # 4: causal striped ring attention, every rank's 8 steps, S = 128k.
    "striped_causal_128k": RingWorkload(
        name="striped_causal_128k", B=1, H=32, D=128, S=131072, cp=8, dtype="bf16", seed=5,
        qk_norm=False, H_total=32, layout="striped", causal=True, ranks=tuple(range(8)),
        variants=("online",)),
    # Contrast of the striped workload (not one of the five): the same causal attention with
    # contiguous shards, where rank r sees r full chunks, its own triangle and cp - 1 - r empty
    # steps, so the work per rank grows with r.
    "contiguous_causal_128k": RingWorkload(
        name="contiguous_causal_128k", B=1, H=32, D=128, S=131072, cp=8, dtype="bf16", seed=5,
        qk_norm=False, H_total=32, layout="contiguous", causal=True, ranks=tuple(range(8)),
        variants=("online",)),
}


def workload(name: str):
    return WORKLOADS[name]
