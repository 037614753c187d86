"""Rank-split additivity on the GPU: the expert-parallel layout of the pages
has each of 8 ranks compute its experts' share of every token's output, and
the shares are summed [sglang PR 47065 "Use the aiter MegaMoE small- and
large-input paths", Motivation].  On one GPU: 64 tokens through all 384
experts at full width, once as the whole layer (384 local slots) and once as
eight 48-slot shares (p0 = 48 r).  The eight bf16 partial outputs must add up
to the whole layer's bf16 output within bf16 rounding of each: bf16 keeps 8
significant bits, so rounding to nearest moves a value by at most 2^-8 of
its rounded magnitude, and |sum_r out_r - out| <= 2^-8 (sum_r |out_r| + |out|)
per element (the float32 sums inside each share differ from the whole
layer's only by float32 roundings, 2^16 times smaller).  Every pair must land
in exactly one share, and the whole layer must match the oracle on sampled
tokens.
"""

import numpy as np
import pytest
import torch

import moe_expert_layer_sigmoid_amd as mx
import synth
from oracle import formats as fm
from oracle import moe as om
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_eight_rank_shares_sum_to_the_whole_layer():
    T, E, ranks = 64, 384, 8
    per_rank = E // ranks
    base = synth.make_sweep(T, with_weights=False)
    _say(f"[case] rank split: T={T}, {E} experts as {ranks} shares of {per_rank}")
    whole = synth.with_replica_map(base, base.rep_count, base.rep_slots, np.arange(E, dtype=np.int32), 0, E,
                                   weights_key=synth.WORKLOADS["sweep"]["weights_key"])
    dw = mx.Dims.of(whole.dims)
    buf = P.upload(whole)                       # 384 packed slots (~9.2 GB)
    res_w = P.run_forward(whole, buf=buf)
    assert res_w["chosen"] == "small_m" and res_w["rows"] == T * dw.k
    outs, counts = [], []
    for r in range(ranks):
        ds = mx.Dims.of(whole.dims, p0=r * per_rank, P_local=per_rank)
        per = [mx.moe_packed_bytes(ds, i) // per_rank for i in range(4)]
        w = [buf[n][r * per_rank * per[i]:(r + 1) * per_rank * per[i]] for i, n in enumerate(("w1", "w1s", "w2", "w2s"))]
        out = torch.full((T, dw.H), -1, dtype=torch.int16, device="cuda")
        hist = torch.zeros(dw.P_total, dtype=torch.int32, device="cuda")
        taps = mx.make_taps(ds)
        mx.moe_forward(ds, buf["x"], buf["logits"], *w, buf["rep_count"], buf["rep_slots"], out, mx.workspace(ds),
                       load_hist=hist, taps=taps)
        torch.cuda.synchronize()
        outs.append(fm.bf16_to_f64(out.cpu().numpy().view(np.uint16)))
        counts.append(taps["counts"].cpu().numpy()[:per_rank])
        assert np.array_equal(hist.cpu().numpy(), res_w["hist"]), f"rank {r}: load record"
    # every pair in exactly one share
    assert np.array_equal(np.concatenate(counts), res_w["counts"])
    full = fm.bf16_to_f64(res_w["out"])
    s = np.sum(outs, axis=0)
    tol = 2.0 ** -8 * (np.sum(np.abs(outs), axis=0) + np.abs(full))
    worst = float(np.max(np.abs(s - full) / np.maximum(tol, 1e-300)))
    _say(f"   sum of shares vs whole: worst |diff| / bound = {worst:.3f}")
    assert np.all(np.abs(s - full) <= tol)
    # the whole layer against the oracle on sampled tokens (unconditioned)
    toks = [0, 21, 42, 63]
    ref = np.stack([om.forward_token(whole, t) for t in toks])
    n2, _ = P.rel_errors(full[toks], ref)
    _say(f"   whole layer vs oracle on {len(toks)} tokens: normwise {n2:.2e}")
    assert n2 <= P.OUT_NORM_TOL
    del buf
    synth.inputs.clear_cache()
    torch.cuda.empty_cache()
