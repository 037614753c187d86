"""Pins of the oracle's EPLB rebalance (new replica map from recorded loads)
and weight migration: hand-worked examples, brute force on tiny inputs,
invariants, and the balance improvement on the skewed workload's shape."""

import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import eplb as oe
from oracle import moe as om
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    cases, cur = [], None
    for line in open(os.path.join(GOLD, "eplb_rebalance.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "name":
            cur = {"name": vals[0], "rep_slots": {}}
        elif key == "end":
            cases.append(cur)
        elif key == "rep_slots":
            cur["rep_slots"][int(vals[0])] = [int(v) for v in vals[1:]]
        else:
            nums = [int(v) for v in vals]
            cur[key] = nums[0] if len(nums) == 1 else np.array(nums)
    return cases


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    rc, rs, se = oe.rebalance(case["hist"], case["slot_expert_old"], case["E"], case["ranks"], case["R_max"])
    assert rc.tolist() == case["rep_count"].tolist()
    assert se.tolist() == case["slot_expert_new"].tolist()
    for e, slots in case["rep_slots"].items():
        assert rs[e, :rc[e]].tolist() == slots
        assert (rs[e, rc[e]:] == -1).all()
    p0, P_local, *src = case["migrate_src"].tolist()
    assert oe.migration_sources(case["slot_expert_old"], se, p0, P_local).tolist() == src


def test_replica_counts_min_max_brute_force():
    """The greedy counts reach the smallest possible largest share L_e / c_e
    over every count vector with 1 <= c_e <= R_max summing to P_total."""
    rng = np.random.default_rng(5)
    for trial in range(200):
        E = int(rng.integers(1, 5))
        R = int(rng.integers(1, 5))
        P = int(rng.integers(E, E * R + 1))
        L = rng.integers(0, 6 if trial % 2 else 50, size=E)
        c = oe.replica_counts(L, P, R)
        assert c.sum() == P and (c >= 1).all() and (c <= R).all()
        best = min(max(Fraction(int(l), int(n)) for l, n in zip(L, cc))
                   for cc in itertools.product(range(1, R + 1), repeat=E) if sum(cc) == P)
        assert max(Fraction(int(l), int(n)) for l, n in zip(L, c)) == best


def test_replica_counts_cap_and_errors():
    assert oe.replica_counts(np.array([100, 1]), 4, 2).tolist() == [2, 2]
    with pytest.raises(ValueError):
        oe.replica_counts(np.array([1, 1]), 5, 2)
    with pytest.raises(ValueError):
        oe.rebalance(np.zeros(6, np.int64), np.arange(6) % 3, 3, 4, 2)   # 6 slots on 4 ranks


def _check_map(rc, rs, se, E, P, ranks):
    assert rc.sum() == P and (rc >= 1).all()
    assert (se >= 0).all() and (se < E).all()
    assert np.array_equal(np.bincount(se, minlength=E), rc)
    for e in range(E):
        sl = rs[e, :rc[e]]
        assert (np.diff(sl) > 0).all() and (se[sl] == e).all()
        assert (rs[e, rc[e]:] == -1).all()


def test_kept_slots_are_maximal_brute_force():
    """Inside each rank, no other assignment of the rank's new experts to its
    slots keeps more slots unchanged (so no avoidable migration)."""
    rng = np.random.default_rng(6)
    for _ in range(60):
        E = int(rng.integers(2, 6))
        ranks = int(rng.integers(1, 4))
        lo = max(1, -(-E // ranks))
        per = int(rng.integers(lo, max(lo, 4) + 1))
        P = ranks * per
        if P < E:
            continue
        R = P
        old = rng.integers(0, E, size=P).astype(np.int32)
        old[:E] = rng.permutation(E)
        hist = rng.integers(0, 40, size=P)
        rc, rs, se = oe.rebalance(hist, old, E, ranks, R)
        _check_map(rc, rs, se, E, P, ranks)
        for r in range(ranks):
            sl = slice(r * per, (r + 1) * per)
            got = int((se[sl] == old[sl]).sum())
            best = max(sum(int(a == b) for a, b in zip(perm, old[sl]))
                       for perm in set(itertools.permutations(se[sl].tolist())))
            assert got == best


def test_uniform_loads_without_redundancy():
    """One rank: every expert keeps its slot (nothing migrates).  Several
    ranks: equal shares are dealt round-robin (expert e to rank e mod ranks)."""
    E = 16
    rc, rs, se = oe.rebalance(np.full(E, 7), np.arange(E, dtype=np.int32), E, 1, 1)
    assert se.tolist() == list(range(E)) and rc.tolist() == [1] * E
    for ranks in (2, 4, 16):
        rc, rs, se = oe.rebalance(np.full(E, 7), np.arange(E, dtype=np.int32), E, ranks, 1)
        per = E // ranks
        assert rc.tolist() == [1] * E
        for r in range(ranks):
            assert sorted(se[r * per:(r + 1) * per].tolist()) == list(range(r, E, ranks))


def test_rank_loads_balanced_on_uniform_loads():
    """Equal loads with E = 2 * P_total / ranks: every rank receives the same
    share sum (list scheduling of equal items)."""
    E, ranks, per = 32, 8, 6
    rc, rs, se = oe.rebalance(np.full(ranks * per, 10), np.arange(ranks * per) % E, E, ranks, 4)
    L = oe.expert_loads(np.full(ranks * per, 10), np.arange(ranks * per) % E, E)
    share = L / rc
    rank_load = [share[se[r * per:(r + 1) * per]].sum() for r in range(ranks)]
    assert max(rank_load) - min(rank_load) <= share.max() + 1e-9


def test_expert_loads_sum_and_migrate():
    rng = np.random.default_rng(7)
    old = rng.integers(-1, 5, size=20).astype(np.int32)
    h = rng.integers(0, 9, size=20)
    L = oe.expert_loads(h, old, 5)
    assert L.sum() == h[old >= 0].sum()
    for e in range(5):
        assert L[e] == sum(int(h[s]) for s in range(20) if old[s] == e)
    slots = rng.integers(0, 255, size=(4, 3, 8)).astype(np.uint8)
    pool = rng.integers(0, 255, size=(5, 3, 8)).astype(np.uint8)
    src = np.array([-1, 4, 0, -1], np.int32)
    out = oe.migrate(slots, pool, src)
    assert np.array_equal(out[0], slots[0]) and np.array_equal(out[3], slots[3])
    assert np.array_equal(out[1], pool[4]) and np.array_equal(out[2], pool[0])


def test_rebalance_improves_skewed_slot_loads():
    """Zipf(1.2) routing over 384 experts with 64 redundant slots on 8 ranks:
    starting from the naive map, one rebalance from a recorded batch lowers the
    largest slot load (and the largest rank load) on a fresh batch."""
    E, k, P, ranks, T = 384, 6, 448, 8, 8192
    rc0, rs0, se0 = synth.naive_replica_map(E, P)
    ids, _ = om.route(synth.skewed_logits(3, 0, T, E, k), k)
    _, hist0 = om.remap_record(ids, rc0, rs0, 0, P)
    assert hist0.sum() == T * k
    rc1, rs1, se1 = oe.rebalance(hist0, se0, E, ranks, 64)
    _check_map(rc1, rs1, se1, E, P, ranks)
    fresh, _ = om.route(synth.skewed_logits(3, 1, T, E, k), k)
    _, before = om.remap_record(fresh, rc0, rs0, T, P)
    _, after = om.remap_record(fresh, rc1, rs1, T, P)
    mx0, mean = oe.slot_loads(before)
    mx1, _ = oe.slot_loads(after)
    assert mx1 < 0.5 * mx0, (mx0, mx1, mean)
    per = P // ranks
    rank = lambda h: h.reshape(ranks, per).sum(1).max()  # noqa: E731
    assert rank(after) < rank(before)
