"""Seeded synthetic inputs for the attention hot path.

This module is shared by the tests, the benchmark and the oracle checks. It only
draws random numbers and shapes them into tensors; it holds none of the attention
arithmetic (no scores, no softmax, no merge, no sharding rule).

Every tensor comes from ``torch.randn`` driven by a ``torch.Generator`` seeded
from the workload seed plus a fixed per-tensor offset, on the device the caller
names. The oracle never regenerates inputs: it reads back the exact tensors that
the GPU path consumed (bf16 and fp32 decode exactly into fp64).
"""

from .configs import (  # noqa: F401
    WORKLOADS,
    RingWorkload,
    DecodeWorkload,
    workload,
)
from .gen import (  # noqa: F401
    normal,
    rms_normed_heads,
    ring_inputs,
    decode_inputs,
    sample_rows,
)
