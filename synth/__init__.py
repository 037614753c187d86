"""Seeded synthetic inputs for the fused MoE expert layer.

This package is shared by the CPU oracle (``oracle/``) and the HIP path's
tests and benchmark.  It only *draws* inputs: router logits, bf16 activations,
MXFP4 expert weights (the checkpoint format the layer consumes), and the EPLB
replica tables.  It holds none of the layer's own arithmetic (routing, remap,
activation quantisation, GEMMs, SwiGLU, combine, EPLB rebalance).  Its
greedy replica map only draws the starting replica table of the skewed
workload from a target popularity; the rebalance from recorded loads is the
method's and is implemented separately by the oracle and the library.
"""

from .inputs import (  # noqa: F401
    Dims,
    Workload,
    SWEEP_T,
    WORKLOADS,
    dims_for,
    make,
    make_ep_shaped,
    make_sweep,
    make_custom,
    naive_replica_map,
    expert_weights,
    gate_weights,
    token_batch,
    with_replica_map,
    skewed_logits,
    sha256,
)
