"""Pins of the oracle's error bounds (oracle.moe gemm_error_bound,
swiglu_error_terms, act_error_bound): the tolerances the GPU parity checks
of GEMM1's requantised act (and of GEMM2's y at the widest rows) rest on.

Each bound is checked against something other than itself:
  * silu's second derivative against finite differences of the oracle's silu
    (the |silu''| <= 1/2 step of the mean value argument);
  * the SwiGLU propagation against the exact float64 change of silu(g) u under
    the worst perturbation on a grid, with one designed case per term that
    fails once that term is left out;
  * the float32 term against a float32 evaluation of silu(g) u step by step
    (the operations the GPU kernels use);
  * the accumulation bound against a float32 emulation of a chain of
    instructions, each off by the full per-instruction allowance in the same
    direction, which also fails once the float32 chain term is left out;
  * act_error_bound end to end on the tiny workload against that emulation
    followed by the float32 SwiGLU.
"""

import numpy as np
import pytest

from oracle import formats as fm
from oracle import moe as om
import synth

TERMS = ("gate", "up", "cross", "curv", "f32")


def _silu2_closed(g):
    s = om.sigmoid(g)
    return s * (1 - s) * (2 + g * (1 - 2 * s))


def test_silu_second_derivative_at_most_half():
    g = np.linspace(-60.0, 60.0, 240001)
    step = 1e-3
    fd = (om.silu(g + step) - 2 * om.silu(g) + om.silu(g - step)) / step ** 2
    cf = _silu2_closed(g)
    assert np.max(np.abs(fd - cf)) < 1e-6            # the closed form is silu''
    assert np.max(np.abs(cf)) <= 0.5 and abs(_silu2_closed(np.array([0.0]))[0] - 0.5) < 1e-15
    assert np.max(np.abs(fd)) <= 0.5 + 1e-6


def _worst_change(g, u, eg, eu, n=401):
    """max over |dg| <= eg, |du| <= eu of |silu(g + dg)(u + du) - silu(g) u|
    (exact float64; act is linear in du, so du = +-eu suffices)."""
    dg = np.linspace(-eg, eg, n)
    base = om.silu(np.array([g]))[0] * u
    best = 0.0
    for du in (-eu, eu):
        best = max(best, float(np.max(np.abs(om.silu(g + dg) * (u + du) - base))))
    return best


def _terms(g, u, eg, eu):
    h = np.array([[g, u]])
    eh = np.array([[eg, eu]])
    return {k: float(v[0, 0]) for k, v in om.swiglu_error_terms(h, eh, 1).items()}


# one case per term: without that term the bound is below the worst change
DESIGNED = {
    "gate": (1.0, 10.0, 1e-3, 0.0),
    "up": (3.0, 0.1, 0.0, 1e-3),
    "cross": (0.0, 0.0, 1e-2, 1e-2),
    "curv": (0.0, 10.0, 0.1, 0.0),
}


@pytest.mark.parametrize("term", sorted(DESIGNED))
def test_swiglu_terms_cover_the_worst_change_and_each_is_needed(term):
    g, u, eg, eu = DESIGNED[term]
    t = _terms(g, u, eg, eu)
    worst = _worst_change(g, u, eg, eu)
    total = sum(t.values())
    assert worst <= total
    assert worst > total - t[term], f"{term}: the bound holds without it"


def test_swiglu_bound_covers_random_perturbations():
    rng = np.random.default_rng(5)
    for _ in range(400):
        g, u = rng.normal(0, 4), rng.normal(0, 4)
        eg, eu = 10.0 ** rng.uniform(-7, -0.5), 10.0 ** rng.uniform(-7, -0.5)
        assert _worst_change(g, u, eg, eu, n=101) <= sum(_terms(g, u, eg, eu).values())


def test_f32_term_covers_float32_evaluation():
    """silu(g) u evaluated in float32 the way the kernels do (g * -log2(e),
    exp2, 1 + e, reciprocal, g * r, times u) from exact gate / up values: only
    the f32 term is non-zero (no accumulation error), and it is needed."""
    rng = np.random.default_rng(6)
    g32 = np.concatenate([np.linspace(-100, 100, 20001), rng.normal(0, 5, 20000)]).astype(np.float32)
    u32 = rng.normal(0, 3, g32.size).astype(np.float32)
    with np.errstate(over="ignore"):
        e = np.exp2(g32 * np.float32(-1.4426950408889634))
        r = np.float32(1.0) / (np.float32(1.0) + e)
        act32 = ((g32 * r) * u32).astype(np.float64)
    g, u = g32.astype(np.float64), u32.astype(np.float64)
    act = om.silu(g) * u
    h = np.stack([g, u], axis=1)
    terms = om.swiglu_error_terms(h, np.zeros_like(h), 1)
    for k in ("gate", "up", "cross", "curv"):
        assert np.all(terms[k] == 0)
    err = np.abs(act32 - act)
    assert np.all(err <= terms["f32"][:, 0])
    assert np.count_nonzero(err) > 1000


def _chain(a, W, rel, sign=1.0):
    """float32 emulation of K/128 chained instructions: each adds the exact sum
    of its 128 products plus sign * rel * (sum of their |products|) to the
    accumulator, then rounds to float32."""
    rows, K = a.shape
    acc = np.zeros((rows, W.shape[0]), np.float32)
    for k0 in range(0, K, 128):
        p = a[:, None, k0:k0 + 128] * W[None, :, k0:k0 + 128]
        s = p.sum(-1) + sign * rel * np.abs(p).sum(-1)
        acc = (acc.astype(np.float64) + s).astype(np.float32)
    return acc.astype(np.float64)


def _operands(rows, outs, K, seed):
    rng = np.random.default_rng(seed)
    q, s = om.quant_blocks(rng.normal(0, 1, (rows, K)))
    a = om.dequant_blocks(q, s)
    w, ws = synth.inputs._encode_mxfp4(rng.normal(0, 0.02, (outs, K)).astype(np.float32))
    return a, fm.dequant_mxfp4(w, ws)


@pytest.mark.parametrize("K", [256, 2048])
def test_gemm_bound_covers_chained_instruction_rounding(K):
    a, W = _operands(16, 64, K, K)
    exact = a @ W.T
    bound = om.gemm_error_bound(a, W)
    mag = np.abs(a) @ np.abs(W).T
    for sign in (1.0, -1.0):
        got = _chain(a, W, om.MFMA_REL, sign)
        assert np.all(np.abs(got - exact) <= bound)
        # without the float32 chain term the bound fails: the roundings add to
        # the instructions' full allowance somewhere
        assert np.any(np.abs(got - exact) > om.MFMA_REL * mag)


def test_act_error_bound_end_to_end_on_the_tiny_workload():
    """GEMM1 by the emulated chain (every instruction off by the full allowance),
    SwiGLU in float32: every act within act_error_bound of the oracle's."""
    wl = synth.make("tiny")
    r = om.forward(wl)
    d = wl.dims
    for s in range(d.P_local):
        lo, hi = int(r["offsets"][s]), int(r["offsets"][s + 1])
        if hi == lo:
            continue
        a = om.dequant_blocks(r["xq"][lo:hi], r["xs"][lo:hi])
        W = fm.dequant_mxfp4(wl.w1[s], wl.w1s[s])
        h32 = _chain(a, W, om.MFMA_REL).astype(np.float32)
        g32, u32 = h32[:, :d.F], h32[:, d.F:]
        rr = np.float32(1.0) / (np.float32(1.0) + np.exp2(g32 * np.float32(-1.4426950408889634)))
        act32 = ((g32 * rr) * u32).astype(np.float64)
        b = om.act_error_bound(a, wl.w1[s], wl.w1s[s], a @ W.T, d.F)
        assert np.all(np.abs(act32 - r["act"][lo:hi]) <= b)
