"""Seeded synthetic inputs for the fused MoE expert layer.

This package is shared by the CPU oracle (``oracle/``) and the HIP path's
tests and benchmark.  It only *draws* inputs: router logits, bf16 activations,
MXFP4 expert weights (the checkpoint format the layer consumes), and the EPLB
replica tables.  It holds none of the layer's own arithmetic (routing, remap,
activation quantisation, GEMMs, SwiGLU, combine).
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
    sha256,
)
