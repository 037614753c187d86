"""GPU parity of the EPLB cycle: record slot loads with the fused forward,
rebalance (host call of the library), migrate the weights on the GPU, and run
the layer again on the new replica table -- each step against the oracle."""

import numpy as np
import pytest
import torch

import moe_expert_layer_sigmoid_amd as mx
import synth
from oracle import eplb as oe
from oracle import formats as fm
from oracle import moe as om
from tests import parity as P
from tests.test_gpu_parity import _big_check, _full_check, _say

pytestmark = pytest.mark.gpu


def _pack(H, F, natural):
    """Packed weights of a stack of experts (the library's repack)."""
    n = natural[0].shape[0]
    d = mx.Dims(T=1, T_max=1, H=H, F=F, E=1, k=1, P_total=n, p0=0, P_local=n, R_max=1)
    return mx.pack_weights(d, *[P.dev(a) for a in natural])


def _cycle(wl0, se0, rc0, rs0, ranks, R_max, p0, P_local, wkey, batch2, path="auto"):
    """Forward on the old map with recording -> rebalance -> migrate -> the
    new map's weights and table.  Returns (migrated packed weights, new map)."""
    d0 = wl0.dims
    res0 = P.run_forward(wl0, path=path, taps=False)
    ref_ids, _ = om.route(wl0.logits, d0.k)
    _, ref_hist = om.remap_record(ref_ids, rc0, rs0, d0.token_id_base, d0.P_total)
    assert np.array_equal(res0["hist"], ref_hist), "recorded loads"
    new = mx.moe_eplb_rebalance(d0.E, d0.P_total, ranks, R_max, res0["hist"], se0)
    ref_new = oe.rebalance(ref_hist, se0, d0.E, ranks, R_max)
    for a, b in zip(new, ref_new):
        assert np.array_equal(a, b), "rebalanced replica table"
    rc1, rs1, se1 = new
    src = oe.migration_sources(se0, se1, p0, P_local)
    _say(f"   rebalanced: {int((src >= 0).sum())} of {P_local} local slots migrate, "
         f"max replicas {int(rc1.max())}")
    # the pool: packed weights of every logical expert a local slot needs
    need = sorted(set(int(e) for e in src if e >= 0))
    assert need, "the skewed loads move at least one local slot"
    packed_need = _pack(d0.H, d0.F, synth.expert_weights(wkey, d0.H, d0.F, need))
    d = mx.Dims.of(d0)
    per = [mx.moe_packed_bytes(d, i) // d.P_local for i in range(4)]
    pool = [torch.zeros(per[i] * d0.E, dtype=torch.uint8, device="cuda") for i in range(4)]
    for j, e in enumerate(need):
        for i in range(4):
            pool[i][e * per[i]:(e + 1) * per[i]] = packed_need[i][j * per[i]:(j + 1) * per[i]]
    slots = P.upload(wl0)
    buf = [slots["w1"], slots["w1s"], slots["w2"], slots["w2s"]]
    before = [b.clone() for b in buf]
    mx.moe_eplb_migrate(d, P.dev(src), d0.E, pool, buf)
    torch.cuda.synchronize()
    # bit-exact: migrated slots hold the pool expert's bytes, kept slots are untouched
    want = _pack(d0.H, d0.F, synth.expert_weights(wkey, d0.H, d0.F, se1[p0:p0 + P_local]))
    for i in range(4):
        assert torch.equal(buf[i], want[i]), f"migrated buffer {i}"
        for s in np.nonzero(src < 0)[0]:
            sl = slice(int(s) * per[i], (int(s) + 1) * per[i])
            assert torch.equal(buf[i][sl], before[i][sl])
    lg, x = batch2
    wl1 = synth.with_replica_map(wl0, rc1, rs1, se1, p0, P_local, wkey, logits=lg, x=x)
    return wl1, dict(x=P.dev(wl1.x.view(np.int16)), logits=P.dev(wl1.logits), w1=buf[0], w1s=buf[1],
                     w2=buf[2], w2s=buf[3], rep_count=P.dev(rc1), rep_slots=P.dev(rs1))


@pytest.mark.parametrize("p0", [0, 6])
def test_eplb_cycle_tiny(p0):
    """8 experts, top-2, Zipf(1.2) routing, 4 redundant slots over 2 ranks of
    6; this GPU holds one rank.  The layer after migration matches the oracle
    on the new table, and its hottest slot carries less load."""
    T, H, F, E, k, seed = 256, 256, 128, 8, 2, 300
    base = synth.make_custom(T=T, H=H, F=F, E=E, k=k, P_local=E, zipf_s=1.2, seed=seed)
    rc0, rs0, se0 = synth.naive_replica_map(E, 12)
    wkey = 1000 + seed
    wl0 = synth.with_replica_map(base, rc0, rs0, se0, p0, 6, wkey)
    _say(f"[case] eplb cycle tiny p0={p0}")
    batch2 = synth.token_batch(seed, 1, T, H, E, k, 1.2)
    wl1, buf = _cycle(wl0, se0, rc0, rs0, 2, 6, p0, 6, wkey, batch2)
    d = wl1.dims
    res = P.run_forward(wl1, buf=buf)
    ref = P.oracle_front(wl1)
    P.check_front(res, ref, d)
    y_c, _ = P.expert_check(wl1, res, ref, range(d.P_local))
    cond = P.conditioned_out(list(range(d.T)), ref, y_c, d)
    P.check_out(res["out"], cond, "conditioned")
    n2, _ = P.rel_errors(fm.bf16_to_f64(res["out"]), om.forward(wl1)["out"])
    assert n2 <= P.OUT_NORM_TOL
    # balance on the second batch: new table vs the naive one
    ids2, _ = om.route(batch2[0], k)
    _, h_old = om.remap_record(ids2, rc0, rs0, 0, 12)
    assert res["hist"].max() < h_old.max(), (res["hist"].max(), h_old.max())


def test_eplb_cycle_448_slots():
    """The skewed workload's shape: 384 experts, top-6 Zipf(1.2) routing over
    8192 tokens, 64 redundant slots on 8 ranks of 56, this GPU rank 0, the
    layer's 7168 x 2048 experts.  Record on the naive map, rebalance, migrate,
    then check the layer on a fresh batch (integer stages in full, GEMM
    stages on sampled slots and tokens)."""
    E, k, T, Pt, ranks = 384, 6, 8192, 448, 8
    wl = synth.make("eplb8192", with_weights=False)
    rc0, rs0, se0 = synth.naive_replica_map(E, Pt)
    wkey = synth.WORKLOADS["eplb8192"]["weights_key"]
    wl0 = synth.with_replica_map(wl, rc0, rs0, se0, 0, 56, wkey)
    _say(f"[case] eplb cycle 448 slots T={T}")
    batch2 = synth.token_batch(synth.WORKLOADS["eplb8192"]["key"], 1, T, wl.dims.H, E, k, 1.2)
    wl1, buf = _cycle(wl0, se0, rc0, rs0, ranks, 64, 0, 56, wkey, batch2)
    res = _big_check(wl1, n_slots=2, n_tokens=12, buf=buf)
    ids2, _ = om.route(batch2[0], k)
    _, h_old = om.remap_record(ids2, rc0, rs0, 0, Pt)
    _say(f"   largest slot load {int(h_old.max())} -> {int(res['hist'].max())} (mean {T * k / Pt:.0f})")
    assert res["hist"].max() < 0.5 * h_old.max()
