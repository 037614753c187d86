"""Pins of the oracle's quantisers, GEMMs, SwiGLU and the whole layer."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as fm
from oracle import moe as om
import synth
import synth.inputs as si

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- O4/O7 quantiser

def test_scale_exponent_is_the_smallest_power():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        np.abs(rng.standard_normal(5000)) * 10.0 ** rng.uniform(-30, 30, 5000),
        448.0 * 2.0 ** np.arange(-60, 60, dtype=np.float64),                # exact boundaries
        np.nextafter(448.0 * 2.0 ** np.arange(-60, 60, dtype=np.float64), np.inf),
        np.nextafter(448.0 * 2.0 ** np.arange(-60, 60, dtype=np.float64), 0),
        2.0 ** np.arange(-100, 100, dtype=np.float64),
    ])
    e = om.scale_exponent(a)
    assert np.all(a <= 448.0 * np.exp2(e.astype(np.float64)))
    assert np.all(a > 448.0 * np.exp2(e.astype(np.float64) - 1))
    assert om.scale_exponent(np.array([0.0]))[0] == 0
    assert om.scale_exponent(np.array([1e-300]))[0] == -127
    assert om.scale_exponent(np.array([448.0]))[0] == 0
    assert om.scale_exponent(np.array([448.5]))[0] == 1


def test_quant_blocks_matches_torch_cast():
    wl = synth.make("tiny", with_weights=False)
    v = fm.bf16_to_f64(wl.x)
    q, s = om.quant_blocks(v)
    e = s.astype(np.int64) - 127
    scaled = np.ldexp(v.reshape(v.shape[0], -1, 128), -e[..., None]).reshape(v.shape)
    ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    # every block's largest element lands in the top binade [256, 448]
    amax_code = fm.dec_e4m3fn(q).reshape(q.shape[0], -1, 128)
    assert np.all(np.abs(amax_code).max(-1) >= 224)


def test_quant_blocks_all_bf16_values_single_element_and_block_edges():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = fm.bf16_to_f64(bits[(bits & 0x7F80) != 0x7F80])
    n = v.size // 128 * 128
    # each value alone in its block: scaled value is v * 2^-e with amax = |v|
    blk = np.zeros((n, 128))
    blk[np.arange(n), np.arange(n) % 128] = v[:n]
    q, s = om.quant_blocks(blk)
    e = s[:, 0].astype(np.int64) - 127
    d = fm.dec_e4m3fn(q[np.arange(n), np.arange(n) % 128]) * np.exp2(e.astype(np.float64))
    nz = v[:n] != 0
    # a block maximum is quantised with relative error <= 2^-4 (half a step of 3 mantissa bits)
    assert np.all(np.abs(d[nz] - v[:n][nz]) <= np.abs(v[:n][nz]) * 2.0 ** -4)
    # edges of a 128-column block: scale is shared, values at both ends
    rows = v[:n].reshape(-1, 128)
    q2, s2 = om.quant_blocks(rows)
    dq = om.dequant_blocks(q2, s2)
    step = np.exp2(s2.astype(np.float64) - 127)[:, :1] * 2.0 ** -9
    amax = np.abs(rows).max(1, keepdims=True)
    rel_ok = np.abs(dq - rows) <= np.maximum(np.abs(rows) * 2.0 ** -4, step / 2)
    assert np.all(rel_ok | (amax == 0))


# ---------------------------------------------------------------- O5-O8 one expert

def _fsum_rows(a, W):
    return np.array([[math.fsum((a[i] * W[j]).tolist()) for j in range(W.shape[0])] for i in range(a.shape[0])])


def test_gemm1_swiglu_against_exact_python_sums():
    rng = np.random.default_rng(6)
    n, H, F = 5, 256, 64
    x = fm.bf16_to_f64(si.f32_to_bf16_bits(rng.standard_normal((n, H)).astype(np.float32)))
    xq, xs = om.quant_blocks(x)
    a = om.dequant_blocks(xq, xs)
    w1, w1s = si._encode_mxfp4((rng.standard_normal((2 * F, H)) * 0.02).astype(np.float32))
    act, h = om.gemm1_swiglu(a, w1, w1s, F)
    W = fm.dequant_mxfp4(w1, w1s)
    exact = _fsum_rows(a, W)                       # products are exact in f64; fsum is exact
    mag = np.abs(a) @ np.abs(W).T
    assert np.all(np.abs(h - exact) <= mag * 2.0 ** -50)
    g, u = exact[:, :F], exact[:, F:]
    want = np.array([[gi / (1 + math.exp(-gi)) * ui for gi, ui in zip(gr, ur)] for gr, ur in zip(g, u)])
    assert np.allclose(act, want, rtol=1e-13, atol=1e-300)


def test_gemm2_against_exact_python_sums():
    rng = np.random.default_rng(7)
    n, H, F = 4, 128, 128
    act = rng.standard_normal((n, F))
    aq, as_ = om.quant_blocks(act)
    ad = om.dequant_blocks(aq, as_)
    w2, w2s = si._encode_mxfp4((rng.standard_normal((H, F)) * 0.02).astype(np.float32))
    y = om.gemm2(ad, w2, w2s)
    exact = _fsum_rows(ad, fm.dequant_mxfp4(w2, w2s))
    assert np.all(np.abs(y - exact) <= (np.abs(ad) @ np.abs(fm.dequant_mxfp4(w2, w2s)).T) * 2.0 ** -50)


def _identity_layer(xval, H=256, F=128, T=3):
    """One expert whose GEMMs copy columns: gate/up row f and down row c one-hot."""
    w1 = np.zeros((1, 2 * F, H // 2), np.uint8)
    for f in range(F):
        for r in (f, F + f):
            w1[0, r, f // 2] = 0x2 << (4 * (f % 2))       # e2m1 1.0 at column f
    w2 = np.zeros((1, H, F // 2), np.uint8)
    for c in range(F):
        w2[0, c, c // 2] = 0x2 << (4 * (c % 2))
    w1s = np.full((1, 2 * F, H // 32), 127, np.uint8)
    w2s = np.full((1, H, F // 32), 127, np.uint8)
    d = synth.Dims(T=T, T_max=T, H=H, F=F, E=1, k=1, P_total=1, p0=0, P_local=1, R_max=1)
    x = si.f32_to_bf16_bits(np.full((T, H), xval, np.float32))
    return synth.Workload(name="identity", dims=d, logits=np.zeros((T, 1), np.float32), x=x,
                          rep_count=np.ones(1, np.int32), rep_slots=np.zeros((1, 1), np.int32),
                          slot_expert=np.zeros(1, np.int32), w1=w1, w1s=w1s, w2=w2, w2s=w2s)


def test_identity_expert_hand_values():
    with open(os.path.join(GOLD, "identity_expert.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert rows
    for xs, acts, lo, hi in rows:
        wl = _identity_layer(float(xs))
        r = om.forward(wl)
        assert np.allclose(r["act"], float(acts), rtol=1e-15)
        assert np.all(r["out"][:, :128] == float(lo)) and np.all(r["out"][:, 128:] == float(hi))
        assert np.all(fm.bf16_to_f64(r["out_bf16"][:, :128]) == float(lo))


def test_zero_experts_give_zero_output():
    wl = synth.make("tiny")
    wl.rep_slots = wl.rep_slots + 100          # every pair lands outside this GPU's slots
    d = wl.dims.replace(P_total=200)
    wl.dims = d
    r = om.forward(wl)
    assert r["offsets"][-1] == 0 and np.all(r["out"] == 0) and np.all(r["out_bf16"] == 0)
    assert r["load_hist"].sum() == d.T * d.k


# ---------------------------------------------------------------- whole layer

def test_layer_second_formulation_per_token():
    """Bucketed O3-O9 equals the per-token sum over its experts, no permutation."""
    wl = synth.make("tiny")
    r = om.forward(wl)
    for t in range(wl.dims.T):
        o = om.forward_token(wl, t)
        scale = np.abs(o).max() + 1e-30
        assert np.allclose(r["out"][t], o, rtol=0, atol=scale * 1e-12), t


def test_layer_invariants_tiny():
    wl = synth.make("tiny")
    d = wl.dims
    r = om.forward(wl)
    assert r["load_hist"].sum() == d.T * d.k
    assert r["counts"].sum() == d.T * d.k                          # all experts local
    assert np.allclose(r["topk_w"].sum(1), 1.0, atol=1e-15)
    assert r["out"].shape == (d.T, d.H) and np.all(np.isfinite(r["out"]))


def test_rank_split_additivity_tiny():
    """Two GPUs holding slots [0,4) and [4,8) produce partial sums that add to the full layer."""
    wl = synth.make("tiny")
    full = om.forward(wl)
    parts = []
    for p0 in (0, 4):
        w = synth.make("tiny")
        d = w.dims.replace(P_local=4, p0=p0)
        w.dims = d
        w.w1, w.w1s, w.w2, w.w2s = (a[p0:p0 + 4] for a in (wl.w1, wl.w1s, wl.w2, wl.w2s))
        parts.append(om.forward(w))
    tot = parts[0]["out"] + parts[1]["out"]
    assert np.allclose(tot, full["out"], rtol=0, atol=1e-12 * np.abs(full["out"]).max())
    b = [fm.bf16_to_f64(p["out_bf16"]) for p in parts]
    bf = fm.bf16_to_f64(full["out_bf16"])
    # three bf16 roundings, each within 2^-8 relative (unit roundoff of an 8-bit significand)
    assert np.all(np.abs(b[0] + b[1] - bf) <= 2.0 ** -8 * (np.abs(b[0]) + np.abs(b[1]) + np.abs(bf)) + 1e-30)


def test_tie_zone_flags_midpoints():
    # block of one value at the amax (scale 2^0 at 448) and a value at a midpoint
    act = np.zeros((1, 128))
    act[0, 0] = 448.0
    act[0, 1] = 1.0625            # midpoint of 1.0 and 1.125
    act[0, 2] = 1.1               # far from a midpoint
    act[0, 3] = 0.5 * 2.0 ** -9   # subnormal midpoint
    elem, blk = om.requant_tie_zone(act, np.full_like(act, 1e-6))
    assert elem[0, 1] and elem[0, 3] and not elem[0, 2]
    assert blk[0, 0]              # amax sits exactly on 448 * 2^0
    act[0, 0] = 300.0
    elem, blk = om.requant_tie_zone(act, np.full_like(act, 1e-6))
    assert not blk[0, 0]
