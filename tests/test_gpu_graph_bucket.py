"""GPU checks of the small-input path with a device token count
(moe_forward_small_m): for every valid count n of a bucket, the first n rows
are bit-identical to moe_forward over those n tokens (itself checked against
the oracle), the other rows are +0, the load record counts only the valid
tokens; and one captured HIP graph replays every n, idle steps included."""

import dataclasses

import numpy as np
import pytest
import torch

import moe_expert_layer_sigmoid_amd as mx
import synth
from oracle import formats as fm
from oracle import moe as om
from tests import parity as P
from tests.test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _prefix(wl, n):
    return dataclasses.replace(wl, dims=wl.dims.replace(T=n, T_max=max(n, 1)), logits=wl.logits[:n], x=wl.x[:n],
                               name=f"{wl.name}_first{n}")


def _eager(wl, buf, n):
    """moe_forward over the first n tokens (SMALL_M): (out bits [n, H], hist)."""
    if n == 0:
        return np.zeros((0, wl.dims.H), np.uint16), np.zeros(wl.dims.P_total, np.int32)
    w = _prefix(wl, n)
    d = mx.Dims.of(w.dims)
    out = torch.empty((n, d.H), dtype=torch.int16, device="cuda")
    hist = torch.zeros(d.P_total, dtype=torch.int32, device="cuda")
    mx.moe_forward(d, buf["x"][:n], buf["logits"][:n], buf["w1"], buf["w1s"], buf["w2"], buf["w2s"],
                   buf["rep_count"], buf["rep_slots"], out, mx.workspace(d), load_hist=hist, path="small_m")
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), hist.cpu().numpy()


def _bucket_case():
    # 64-token bucket, 384 experts top-6 with 48 local slots at a small width
    return synth.make_custom(T=64, H=512, F=256, E=384, k=6, P_local=48, seed=410)


@pytest.mark.parametrize("n", [64, 37, 16, 1, 0])
def test_bucket_matches_eager_prefix(n):
    wl = _bucket_case()
    _say(f"[case] bucket 64, valid {n}")
    buf = P.upload(wl)
    d = mx.Dims.of(wl.dims)
    nt = torch.tensor([n], dtype=torch.int32, device="cuda")
    out = torch.full((d.T, d.H), -1, dtype=torch.int16, device="cuda")
    hist = torch.zeros(d.P_total, dtype=torch.int32, device="cuda")
    mx.moe_forward_small_m(d, nt, buf["x"], buf["logits"], buf["w1"], buf["w1s"], buf["w2"], buf["w2s"],
                           buf["rep_count"], buf["rep_slots"], out, mx.workspace(d), load_hist=hist)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    ref_out, ref_hist = _eager(wl, buf, n)
    assert np.array_equal(got[:n], ref_out), "valid rows differ from moe_forward over the same tokens"
    assert np.all(got[n:] == 0), "rows past the device count must be +0"
    assert np.array_equal(hist.cpu().numpy(), ref_hist)
    if n:
        ids, _ = om.route(wl.logits[:n], 6)
        _, o_hist = om.remap_record(ids, wl.rep_count, wl.rep_slots, 0, d.P_total)
        assert np.array_equal(ref_hist, o_hist)
        n2, _ = P.rel_errors(fm.bf16_to_f64(got[:n]), om.forward(_prefix(wl, n))["out"])
        assert n2 <= P.OUT_NORM_TOL
        _say(f"   ok: normwise vs oracle {n2:.2e}")


def test_captured_graph_replays_every_count():
    """Capture once at a 64-token bucket; replay with n = 64, 37, 0 (idle),
    1, 50, with eager work and synchronisation between replays; every replay
    equals the eager call for its n."""
    wl = _bucket_case()
    buf = P.upload(wl)
    d = mx.Dims.of(wl.dims)
    nt = torch.tensor([d.T], dtype=torch.int32, device="cuda")
    out = torch.full((d.T, d.H), -1, dtype=torch.int16, device="cuda")
    hist = torch.zeros(d.P_total, dtype=torch.int32, device="cuda")
    ws = mx.workspace(d)
    args = (d, nt, buf["x"], buf["logits"], buf["w1"], buf["w1s"], buf["w2"], buf["w2s"], buf["rep_count"],
            buf["rep_slots"], out, ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        mx.moe_forward_small_m(*args, load_hist=hist)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.moe_forward_small_m(*args, load_hist=hist)
    torch.cuda.synchronize()
    for n in (64, 37, 0, 1, 50):
        _say(f"[case] graph replay, valid {n}")
        nt.fill_(n)
        hist.zero_()
        out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        ref_out, ref_hist = _eager(wl, buf, n)
        assert np.array_equal(got[:n], ref_out), f"replay with {n} valid tokens"
        assert np.all(got[n:] == 0)
        assert np.array_equal(hist.cpu().numpy(), ref_hist)
        _ = torch.randn(1000, device="cuda").sum().item()  # eager work between replays
    _say("   ok: every replay equals the eager call")


def test_bucket_rejects_bad_arguments():
    """Capacity above the small-input limit (1024 tokens): an error before any launch."""
    wl = _bucket_case()
    buf = P.upload(wl)
    big = mx.Dims.of(wl.dims, T=1025, T_max=1025)
    x = torch.zeros((1025, big.H), dtype=torch.int16, device="cuda")
    lg = torch.zeros((1025, big.E), dtype=torch.float32, device="cuda")
    out = torch.empty((1025, big.H), dtype=torch.int16, device="cuda")
    with pytest.raises(mx.MoeError) as e:
        mx.moe_forward_small_m(big, torch.zeros(1, dtype=torch.int32, device="cuda"), x, lg, buf["w1"], buf["w1s"],
                               buf["w2"], buf["w2s"], buf["rep_count"], buf["rep_slots"], out, mx.workspace(big))
    assert e.value.code == -2
