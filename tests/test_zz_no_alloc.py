"""The allocation-free entry point, moe_forward_noalloc, against moe_forward.

moe_forward_noalloc runs moe_forward's kernels with the library's fixed
per-GPU scratch as the workspace.  On the same inputs both must give the
same output bits and the same load record; two calls in a row, the second
with a smaller input, check that what the first call left in the shared
scratch does not reach the second.
"""

import numpy as np
import pytest
import torch

import moe_expert_layer_sigmoid_amd as mx
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _both(wl, buf, path):
    """(out, hist, chosen) of moe_forward and of moe_forward_noalloc."""
    d = mx.Dims.of(wl.dims)
    x = P.dev(wl.x.view(np.int16))
    lg = P.dev(wl.logits)
    res = []
    for noalloc in (False, True):
        out = torch.full((d.T, d.H), -1, dtype=torch.int16, device="cuda")
        hist = torch.zeros(d.P_total, dtype=torch.int32, device="cuda")
        args = (d, x, lg, buf["w1"], buf["w1s"], buf["w2"], buf["w2s"], buf["rep_count"], buf["rep_slots"], out)
        if noalloc:
            chosen = mx.moe_forward_noalloc(*args, load_hist=hist, path=path)
        else:
            chosen = mx.moe_forward(*args, mx.workspace(d), load_hist=hist, path=path)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), hist.cpu().numpy(), chosen))
    return res


def _check(wl, buf, path="auto"):
    d = wl.dims
    _say(f"[case] noalloc {wl.name} T={d.T} H={d.H} F={d.F} P_local={d.P_local} path={path}")
    (o1, h1, c1), (o2, h2, c2) = _both(wl, buf, path)
    assert c1 == c2
    assert np.array_equal(h1, h2), "load record differs"
    assert np.array_equal(o1, o2), "output differs"
    assert h2.sum() == d.T * d.k
    _say(f"   ok: path {c2}, identical output and load record")
    return c2


def test_noalloc_decode_share_then_fewer_tokens():
    # the 512-token decode share (the benchmark workload), then 64 tokens on
    # the same experts: the second call runs on what the first left behind
    big = synth.make("decode512")
    buf = P.upload(big)
    assert _check(big, buf) == "small_m"
    small = synth.make_sweep(64)
    assert _check(small, buf) == "small_m"


def test_noalloc_large_input_path_then_smaller():
    # the bucketed path with the persistent tiled GEMMs, then a smaller call
    big = synth.make_custom(T=1000, H=512, F=1024, E=16, k=4, P_local=8, p0=4, seed=22)
    buf = P.upload(big)
    assert _check(big, buf, "large_m") == "large_m"
    small = synth.make_custom(T=300, H=512, F=1024, E=16, k=4, P_local=8, p0=4, seed=22)
    assert _check(small, buf, "large_m") == "large_m"


def test_noalloc_rejects_dims_beyond_its_scratch():
    wl = synth.make_custom(T=4, H=256, F=128, E=8, k=2, P_local=8, seed=16)
    buf = P.upload(wl)
    d = mx.Dims.of(wl.dims, H=7168, F=2048, T_max=4096)
    assert mx.moe_workspace_bytes(d) > mx.NOALLOC_SCRATCH_BYTES
    out = torch.full((4, 7168), 7, dtype=torch.int16, device="cuda")
    packed = [torch.zeros(mx.moe_packed_bytes(d, i), dtype=torch.uint8, device="cuda") for i in range(4)]
    with pytest.raises(mx.MoeError) as e:
        mx.moe_forward_noalloc(d, P.dev(np.zeros((4, 7168), np.int16)), buf["logits"], *packed,
                               buf["rep_count"], buf["rep_slots"], out)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert torch.all(out == 7)
