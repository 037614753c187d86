"""Pins of the oracle's router projection (logits = x W_gate^T from bf16
operands): exact rational sums, one-hot closed forms, torch's float64 matmul,
and the error-scale helper."""

from fractions import Fraction

import numpy as np
import torch

from oracle import formats as fm
from oracle import router as orr
import synth


def _bf16(v):
    return synth.inputs.f32_to_bf16_bits(np.asarray(v, np.float32))


def test_exact_rational_sums_small():
    rng = np.random.default_rng(21)
    x = _bf16(rng.standard_normal((3, 128)) * 3)
    w = _bf16(rng.standard_normal((5, 128)) * 0.1)
    got = orr.logits(x, w)
    xf, wf = fm.bf16_to_f64(x), fm.bf16_to_f64(w)
    for t in range(3):
        for e in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[t], wf[e]))
            scale = float(sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(xf[t], wf[e])))
            assert abs(float(exact) - got[t, e]) <= 2.0 ** -50 * scale


def test_one_hot_closed_forms():
    H, E = 256, 8
    w = _bf16(np.random.default_rng(3).standard_normal((E, H)))
    x = np.zeros((H, H), np.float32)
    np.fill_diagonal(x, 1.0)
    got = orr.logits(_bf16(x), w)
    assert np.array_equal(got, fm.bf16_to_f64(w).T)          # x = e_k picks column k
    x2 = np.zeros((1, H), np.float32)
    x2[0, 5], x2[0, 9] = 2.0, -0.5
    assert np.array_equal(orr.logits(_bf16(x2), w)[0], 2.0 * fm.bf16_to_f64(w)[:, 5] - 0.5 * fm.bf16_to_f64(w)[:, 9])


def test_matches_torch_float64_matmul():
    x = synth.make("tiny").x
    w = synth.gate_weights(0, 8, 256)
    ref = torch.from_numpy(fm.bf16_to_f64(x)) @ torch.from_numpy(fm.bf16_to_f64(w)).T
    assert np.allclose(orr.logits(x, w), ref.numpy(), rtol=0, atol=1e-12)
    # bf16 -> f64 decoding agrees with torch's bfloat16
    tb = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(fm.bf16_to_f64(x), tb)


def test_abs_products_and_logit_scale():
    x = synth.make("tiny").x
    w = synth.gate_weights(0, 8, 256)
    lg = orr.logits(x, w)
    ap = orr.abs_products(x, w)
    assert np.all(np.abs(lg) <= ap + 1e-12)
    # N(0, 1/H) gate rows: logits of N(0, 1) activations have a standard deviation near 1
    assert 0.8 < lg.std() < 1.2
