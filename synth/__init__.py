"""Seeded synthetic inputs for the TokenGate gated-prefill path.

This package only draws random numbers and lays them out. It holds none of the
method's arithmetic (no scoring, selection, compaction, projection or attention) and is the
one module that both the oracle-side tests and the HIP-side callers share.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    EXTRA,
    Workload,
    WorkloadSpec,
    attention_inputs,
    dense_attention_inputs,
    layer_weights,
    make_workload,
    qkv_weights,
    spec,
    with_overrides,
)
