"""The library's EPLB rebalance (a host call of libmoe, no GPU needed) against
the oracle: bit-exact replica tables on the hand-worked examples, on random
shapes and on the skewed 448-slot workload; invalid arguments are rejected."""

import os

import numpy as np
import pytest

import moe_expert_layer_sigmoid_amd as mx
import synth
from oracle import eplb as oe
from oracle import moe as om
from tests.test_oracle_eplb import _golden

pytestmark = pytest.mark.skipif(not os.path.exists(mx.LIB_PATH), reason="libmoe.so not built")


def _same(a, b):
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x), np.asarray(y))


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    P = len(case["slot_expert_old"])
    got = mx.moe_eplb_rebalance(case["E"], P, case["ranks"], case["R_max"], case["hist"], case["slot_expert_old"])
    assert got[0].tolist() == case["rep_count"].tolist()
    assert got[2].tolist() == case["slot_expert_new"].tolist()
    _same(got, oe.rebalance(case["hist"], case["slot_expert_old"], case["E"], case["ranks"], case["R_max"]))


def test_random_shapes_bit_exact():
    rng = np.random.default_rng(11)
    for trial in range(400):
        E = int(rng.integers(1, 40))
        ranks = int(rng.integers(1, 9))
        lo = -(-E // ranks)
        P = ranks * int(rng.integers(lo, lo + 6))
        R = int(rng.integers(-(-P // E), min(64, P) + 1))
        old = rng.integers(-1, E, size=P).astype(np.int32)
        hist = rng.integers(0, (3, 100, 100000)[trial % 3], size=P).astype(np.int32)
        if trial % 7 == 0:
            hist[:] = 5
        _same(mx.moe_eplb_rebalance(E, P, ranks, R, hist, old), oe.rebalance(hist, old, E, ranks, R))


def test_skewed_448_slots_bit_exact():
    E, k, P, T = 384, 6, 448, 8192
    rc0, rs0, se0 = synth.naive_replica_map(E, P)
    ids, _ = om.route(synth.skewed_logits(3, 0, T, E, k), k)
    _, hist = om.remap_record(ids, rc0, rs0, 0, P)
    _same(mx.moe_eplb_rebalance(E, P, 8, 64, hist, se0), oe.rebalance(hist, se0, E, 8, 64))


def test_invalid_arguments():
    h = np.ones(8, np.int32)
    old = np.arange(8, dtype=np.int32) % 4
    for args in ((4, 8, 3, 4), (9, 8, 1, 4), (4, 8, 2, 1), (0, 8, 1, 4), (4, 8, 0, 4)):
        with pytest.raises(mx.MoeError):
            mx.moe_eplb_rebalance(*args, h, old)
    with pytest.raises(mx.MoeError):
        mx.moe_eplb_rebalance(4, 8, 2, 4, -h, old)
    with pytest.raises(mx.MoeError):
        mx.moe_eplb_rebalance(4, 8, 2, 4, h, old + 4)
