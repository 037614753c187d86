"""Plain CPU oracle of the router projection in front of routing: the router
logits of each token from its activations and the gate weights.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

What the pages fix: the model's gate (router) weights are stored in BF16
[InferenceX PR 3430 "[AMD][MI35X] 0926 DSV4 sglang mtp agentic", Additional
detail section, draft precision]; routing picks the top-6 experts of each
token from the router's scores [sglang PR 35619 "Aiter/FlyDSL MegaMoEv2
backend for DeepSeek-V4", "Four settings that silently break it", item 2].
Reading taken: logits = x W_gate^T, with x the layer's bf16 input [T, H] and
W_gate bf16 [E, H] (one row per logical expert, no bias), accumulated in
float64 here (each bf16 x bf16 product is exact in float64).

Parity: pinned by CPU tests against exact rational sums on small inputs,
one-hot closed forms and torch's float64 matmul.
"""

from __future__ import annotations

import numpy as np

from . import formats as fm


def logits(x_bits: np.ndarray, wg_bits: np.ndarray) -> np.ndarray:
    """float64 [T, E] = dequantised x [T, H] times dequantised W_gate [E, H]^T."""
    x = fm.bf16_to_f64(x_bits)
    w = fm.bf16_to_f64(wg_bits)
    return x @ w.T


def abs_products(x_bits: np.ndarray, wg_bits: np.ndarray) -> np.ndarray:
    """sum_k |x_tk| |w_ek| (float64 [T, E]): the scale of the rounding error
    of any float accumulation of the logit sums."""
    return np.abs(fm.bf16_to_f64(x_bits)) @ np.abs(fm.bf16_to_f64(wg_bits)).T
