"""Plain CPU oracle of the a16w4 variant of the layer: bf16 activations on
MXFP4 experts, no activation quantisation.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

What the pages fix: besides the EP arm's a8w4 MegaMoE, the other arms run
the MXFP4 experts with the default bf16 activations [InferenceX PR 3430
"[AMD][MI35X] 0926 DSV4 sglang mtp agentic", Additional detail section,
draft precision].  Readings taken (the pages give no formula): GEMM1 takes
the bf16 input rows as they are (exact in float64); SwiGLU as in the a8w4
layer; the act is rounded to bf16 (nearest, ties to even) before GEMM2, the
activation dtype of this variant; GEMM2 and the routing-weighted combine as
in the a8w4 layer.  Routing, remap, record and buckets are the a8w4 layer's.

Parity: pinned by CPU tests -- hand-computed identity-expert outputs
(``tests/golden/identity_expert_a16w4.txt``), a per-token second
formulation without buckets, and the shared GEMM / SwiGLU / bf16 pins.
"""

from __future__ import annotations

from typing import Dict

import numpy as np

from . import formats as fm
from . import moe as om


def expert_rows(x_rows: np.ndarray, w1, w1s, w2, w2s, F: int) -> Dict[str, np.ndarray]:
    """GEMM1 + SwiGLU on bf16 rows (float64 values), act -> bf16, GEMM2.
    Returns act (float64), act_bf16 (bits) and y (float64)."""
    act, h = om.gemm1_swiglu(x_rows, w1, w1s, F)
    act_b = fm.f64_to_bf16_rne(act)
    y = om.gemm2(fm.bf16_to_f64(act_b), w2, w2s)
    return dict(act=act, h=h, act_bf16=act_b, y=y)


def forward(wl) -> Dict[str, np.ndarray]:
    """The whole a16w4 layer for a ``synth.Workload`` (its MXFP4 weights and
    bf16 inputs).  Returns the routing / bucket stages, act, act_bf16, y, out
    (float64) and out_bf16."""
    d = wl.dims
    T, H, F, k = d.T, d.H, d.F, d.k
    ids, w = om.route(wl.logits, k)
    phys, hist = om.remap_record(ids, wl.rep_count, wl.rep_slots, d.token_id_base, d.P_total)
    counts, offsets, row_of_pair, pair_of_row = om.buckets(phys, d.p0, d.P_local)
    rows = int(offsets[-1])
    xv = fm.bf16_to_f64(wl.x)
    x_rows = xv[pair_of_row // k]
    act = np.zeros((rows, F))
    act_b = np.zeros((rows, F), np.uint16)
    y = np.zeros((rows, H))
    for s in range(d.P_local):
        lo, hi = int(offsets[s]), int(offsets[s + 1])
        if hi == lo:
            continue
        r = expert_rows(x_rows[lo:hi], wl.w1[s], wl.w1s[s], wl.w2[s], wl.w2s[s], F)
        act[lo:hi], act_b[lo:hi], y[lo:hi] = r["act"], r["act_bf16"], r["y"]
    out = om.combine(y, row_of_pair, w, T, k, H)
    return dict(topk_ids=ids, topk_w=w, phys_ids=phys, load_hist=hist, counts=counts, offsets=offsets,
                row_of_pair=row_of_pair, pair_of_row=pair_of_row, act=act, act_bf16=act_b, y=y, out=out,
                out_bf16=fm.f64_to_bf16_rne(out))


def forward_token(wl, t: int) -> np.ndarray:
    """Output row of token t computed on its own, no buckets (a second
    formulation): sum over its local pairs of w_tj * expert(x_t)."""
    d = wl.dims
    ids, w = om.route(wl.logits[t:t + 1], d.k)
    phys, _ = om.remap_record(ids, wl.rep_count, wl.rep_slots, d.token_id_base + t, d.P_total)
    x = fm.bf16_to_f64(wl.x[t:t + 1])
    out = np.zeros(d.H)
    for j in range(d.k):
        p = int(phys[0, j])
        if not (d.p0 <= p < d.p0 + d.P_local):
            continue
        s = p - d.p0
        out += w[0, j] * expert_rows(x, wl.w1[s], wl.w1s[s], wl.w2[s], wl.w2s[s], d.F)["y"][0]
    return out


def act_error_bound(x_rows: np.ndarray, w1, w1s, h: np.ndarray, F: int, rel: float) -> np.ndarray:
    """Bound on |act_gpu - act| (before the bf16 rounding) from an
    accumulation error of ``rel`` times the sum of absolute products in each
    GEMM1 output, carried through SwiGLU as in the a8w4 layer
    (oracle.moe.swiglu_error_terms)."""
    W = fm.dequant_mxfp4(w1, w1s)
    e = rel * (np.abs(x_rows) @ np.abs(W).T)
    return sum(om.swiglu_error_terms(h, e, F).values())
