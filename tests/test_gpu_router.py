"""GPU parity of the router projection (moe_router_logits) against the
oracle: logits within the f32 accumulation bound of the float64 sums, the
routing decided on those f32 logits bit-identical to the oracle's routing of
the same values, and the whole layer fed by them."""

import dataclasses

import numpy as np
import pytest
import torch

import moe_expert_layer_sigmoid_amd as mx
import synth
from oracle import moe as om
from oracle import router as orr
from tests import parity as P
from tests.test_gpu_parity import _full_check, _say

pytestmark = pytest.mark.gpu

# f32 accumulation of K = H products: H/32 MFMA steps plus at most 16 split
# partials.  The instruction need not round its 32 products once (gfx950's
# block-scaled fp8 MFMA measurably does not), so up to 4 roundings per step are
# allowed, each at most 2^-24 of the running sum of magnitudes:
# |logit - exact| <= (4 H/32 + 16) 2^-24 sum_k |x_k w_k|.
def _bound(H):
    return (4 * H / 32 + 16) * 2.0 ** -24


def _run(T, H, E, key=7, T_max=None):
    x = synth.inputs.f32_to_bf16_bits(np.random.default_rng((key, T, H, E)).standard_normal((T, H)).astype(np.float32))
    wg = synth.gate_weights(key, E, H)
    d = mx.Dims(T=T, T_max=T_max or T, H=H, F=128, E=E, k=min(6, E), P_total=E, p0=0, P_local=E, R_max=1)
    lg = torch.full((max(T, 1), E), float("nan"), dtype=torch.float32, device="cuda")
    mx.moe_router_logits(d, P.dev(x.view(np.int16)), P.dev(wg.view(np.int16)), lg, mx.router_workspace(d))
    torch.cuda.synchronize()
    return x, wg, lg.cpu().numpy()[:T]


def _check_logits(x, wg, got, H):
    ref = orr.logits(x, wg)
    scale = orr.abs_products(x, wg)
    err = np.abs(got.astype(np.float64) - ref)
    worst = float((err / np.maximum(scale, 1e-300)).max()) if err.size else 0.0
    assert np.all(np.isfinite(got))
    assert np.all(err <= _bound(H) * scale), f"logit error {worst:.3g} of sum |x w|"
    return ref, worst


@pytest.mark.parametrize("T,H,E", [(64, 256, 8), (1, 256, 8), (200, 384, 13), (37, 128, 1024),
                                   (3000, 640, 96), (2048, 7168, 384), (5000, 384, 200)])
def test_router_logits_small_and_ragged(T, H, E):
    _say(f"[case] router T={T} H={H} E={E}")
    x, wg, got = _run(T, H, E)
    _, worst = _check_logits(x, wg, got, H)
    _say(f"   ok: worst logit error {worst:.2e} of sum |x w|")


@pytest.mark.parametrize("T", [512, 8192])
def test_router_full_size_and_routing(T):
    """Decode and prefill shares' router (d_model 7168, 384 experts): every
    logit within the bound; top-6 on the GPU's logits (moe_route) equal to the
    oracle's top-6 of the same f32 values, and equal to the float64 logits'
    top-6 wherever the k-th and (k+1)-th logits are further apart than the
    accumulation bound."""
    H, E, k = 7168, 384, 6
    _say(f"[case] router T={T} H={H} E={E}")
    x, wg, got = _run(T, H, E, key=11)
    ref, worst = _check_logits(x, wg, got, H)
    d = mx.Dims(T=T, T_max=T, H=H, F=2048, E=E, k=k, P_total=E, p0=0, P_local=48, R_max=1)
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    mx.moe_route(d, P.dev(got), ids, w)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy().reshape(T, k)
    o_ids, _ = om.route(got, k)
    assert np.array_equal(ids, o_ids), "routing of the GPU's logits"
    f_ids, _ = om.route(ref.astype(np.float32), k)
    srt = -np.sort(-ref, axis=1)
    gap = srt[:, k - 1] - srt[:, k]
    tol = 2 * _bound(H) * orr.abs_products(x, wg).max(axis=1)
    differ = np.nonzero((np.sort(ids, 1) != np.sort(f_ids, 1)).any(1))[0]
    assert np.all(gap[differ] <= tol[differ]), "top-k set differs away from a near tie"
    _say(f"   ok: worst logit error {worst:.2e}; {len(differ)} of {T} tokens change their expert set "
         f"at a near tie")


def test_router_feeds_the_layer():
    """The tiny layer with its router logits produced on the GPU: the whole
    forward checked stage by stage against the oracle given those logits."""
    wl = synth.make("tiny")
    d = mx.Dims.of(wl.dims)
    wg = synth.gate_weights(0, d.E, d.H)
    lg = torch.empty((d.T, d.E), dtype=torch.float32, device="cuda")
    mx.moe_router_logits(d, P.dev(wl.x.view(np.int16)), P.dev(wg.view(np.int16)), lg, mx.router_workspace(d))
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    _check_logits(wl.x, wg, got, d.H)
    _full_check(dataclasses.replace(wl, logits=got, name="tiny_router"))


def test_router_zero_tokens():
    d = mx.Dims(T=0, T_max=16, H=256, F=128, E=8, k=2, P_total=8, p0=0, P_local=8, R_max=1)
    lg = torch.full((1, 8), 7.0, device="cuda")
    x = torch.zeros((1, 256), dtype=torch.int16, device="cuda")
    wg = torch.zeros((8, 256), dtype=torch.int16, device="cuda")
    mx.moe_router_logits(d, x, wg, lg, mx.router_workspace(d))
    torch.cuda.synchronize()
    assert torch.all(lg == 7.0)
