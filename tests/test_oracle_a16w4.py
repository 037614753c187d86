"""Pins of the oracle's a16w4 variant: hand-computed identity-expert values,
a per-token second formulation, the bf16 act rounding, and its reduction to
plain products on bf16 inputs."""

import os

import numpy as np

from oracle import a16w4 as oa
from oracle import formats as fm
from oracle import moe as om
import synth
from tests.test_oracle_layer import _identity_layer

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_identity_expert_hand_values():
    with open(os.path.join(GOLD, "identity_expert_a16w4.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for xs, acts, lo, hi in rows:
        r = oa.forward(_identity_layer(float(xs)))
        assert np.allclose(r["act"], float(acts), rtol=1e-15)
        assert np.all(r["out"][:, :128] == float(lo)) and np.all(r["out"][:, 128:] == float(hi))
        assert np.all(fm.bf16_to_f64(r["out_bf16"][:, :128]) == float(lo))


def test_per_token_formulation_equals_buckets():
    wl = synth.make("tiny")
    r = oa.forward(wl)
    for t in range(wl.dims.T):
        assert np.array_equal(oa.forward_token(wl, t), r["out"][t])


def test_act_is_bf16_of_swiglu_and_matches_torch_rounding():
    import torch
    wl = synth.make("tiny")
    r = oa.forward(wl)
    tb = torch.from_numpy(r["act"]).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(r["act_bf16"], tb)
    assert np.array_equal(r["topk_ids"], om.forward(wl)["topk_ids"])


def test_no_quantisation_of_the_input():
    """A bf16 input that fp8 cannot hold (8 significant bits; e4m3 keeps 4)
    passes GEMM1 unchanged: a single identity column gives silu(x) x of the
    exact bf16 value."""
    x = 1.0 + 2.0 ** -7                 # exact in bf16, not in e4m3
    wl = _identity_layer(x)
    r = oa.forward(wl)
    s = 1.0 / (1.0 + np.exp(-x))
    assert np.allclose(r["act"], x * s * x, rtol=1e-15)
    a8 = om.forward(wl)
    assert not np.allclose(a8["act"], r["act"], rtol=1e-6)   # the a8w4 layer rounds x to fp8 first


def test_act_error_bound_covers_f32_accumulation():
    """An f32 evaluation of GEMM1 (BLAS sgemm, K = 256: error below 256 * 2^-24
    of the sum of absolute products) stays inside the bound at rel = 2^-15."""
    wl = synth.make("tiny")
    r = oa.forward(wl)
    d = wl.dims
    xr = fm.bf16_to_f64(wl.x)[r["pair_of_row"] // d.k]
    for s in range(d.P_local):
        lo, hi = int(r["offsets"][s]), int(r["offsets"][s + 1])
        if hi == lo:
            continue
        W = fm.dequant_mxfp4(wl.w1[s], wl.w1s[s])
        h32 = (xr[lo:hi].astype(np.float32) @ W.T.astype(np.float32)).astype(np.float64)
        act32 = om.silu(h32[:, :d.F]) * h32[:, d.F:]
        h = om.gemm1_swiglu(xr[lo:hi], wl.w1[s], wl.w1s[s], d.F)[1]
        b = oa.act_error_bound(xr[lo:hi], wl.w1[s], wl.w1s[s], h, d.F, 2.0 ** -15)
        assert np.all(np.abs(act32 - r["act"][lo:hi]) <= b)
