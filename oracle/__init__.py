"""fp64 CPU oracle for context-parallel attention with log-sum-exp merging.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP path
(no kernels, helpers, tables or constants), and the HIP path never calls it.

What it computes, and where the pages define it:
- ``attention``: plain softmax attention of a query shard against keys, with the
  per-row log-sum-exp (natural log). This is the always-correct path that the
  context-parallelism page keeps as its fallback (full K/V all-gather, then local
  attention), and that the kernel reference page ("Adapting this kernel",
  validation) says to compare against.
- ``attention.merge_lse``: the DCP page's decode compute pattern, steps 4-7: each
  partial's LSE, the global LSE, weights exp(local_lse - global_lse), weighted sum.
- ``attention.const_max``: the kernel reference page's const-max method: the
  per-row bound c_i = scale * |q_i| * max_j |k_j| ("Picking a max that is safe
  without measuring it"), the pure-addition fold over ring steps ("A static bound
  makes the ring reduction pure addition"), one normalisation with the row sum
  clamped at 1e-37 ("Accumulate, then normalize once"), and lse = c + log(sum)
  (Interface, ``training``). ``const_max_sink_robust``: the same with a handful of
  huge-norm keys taken out of the bound and attended exactly ("Adapting this kernel").
- ``sharding``: contiguous and striped ring sharding (Striped Attention on the
  sequence-sharding survey page; ring schedule from the kernel reference page's
  Overview figure) and the DCP interleave rules (DCP page: local_filled
  computation, dcp_active_mask, slot mapping, segmented attention positions).

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, invariants and the pages' printed integer examples; none is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    SUM_CLAMP,
    to_f64,
    default_scale,
    attention,
    attention_heads,
    merge_lse,
    const_max,
    const_max_bound,
    const_max_sink_robust,
    key_sinks,
)
from .sharding import (  # noqa: F401
    contiguous_tokens,
    striped_tokens,
    ring_source_rank,
    causal_allowed,
    dcp_shard_of_position,
    dcp_local_filled,
    dcp_active_owner,
    dcp_prefill_prior_global_position,
)
from .dcp import (  # noqa: F401
    decode_shard_partial,
    decode_shard_partial_active,
    decode_full,
    segmented_attention_partial,
)
