"""Plain CPU oracle of the EPLB rebalance: a new replica map from the recorded
per-physical-slot load histogram, and the weight migration it implies.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

What the pages fix: EPLB runs with a number of redundant physical experts
and rebalances every N steps (200 or 320) from the loads that the fused
remap/record step counts; rebalancing needs the statistics recorder
[sglang PR 35619 "Aiter/FlyDSL MegaMoEv2 backend for DeepSeek-V4", Summary,
reviewer reproduction, "Four settings that silently break it" item 4]; the
runs compare naive and biased placements and check that rebalancing and
migrations actually happen [FlyDSL issue 978 "Investigate MegaMoEV2
end-to-end throughput gap vs V1 on 8xMI355X", Benchmark plan, Data-quality
gates].  The pages give no placement algorithm.  Reading taken here (the
plainest greedy one, in four steps):

1. logical load L_e = sum of the histogram over the slots that held e;
2. replica counts: every expert starts with one; P_total - E times, the
   expert with the largest L_e / c_e among those below the replica cap gets
   one more (equal shares: the lower e).  Shares are compared exactly;
3. replicas in descending L_e / c_e (then e, then replica index) go one by
   one to the rank with the least load (sum of the f64 shares L_e / c_e
   placed on it, added in placement order) among ranks with a free slot,
   preferring ranks that do not hold e yet (then the lower rank);
4. inside a rank, a replica of e keeps a slot of that rank that held e in
   the old map (the lowest such slot first), so that it needs no migration;
   the other replicas take the rank's remaining slots in ascending order,
   in placement order.
rep_slots[e] lists e's slots in ascending order (the remap picks replica
fmix32(token id) mod c_e of that list).

Parity: pinned by CPU tests against brute force (min-max optimality of the
replica counts, maximal number of kept slots inside each rank), invariants
and a hand-worked example (``tests/golden/eplb_rebalance.txt``).
"""

from __future__ import annotations

from fractions import Fraction
from typing import Tuple

import numpy as np


def expert_loads(hist: np.ndarray, slot_expert: np.ndarray, E: int) -> np.ndarray:
    """L_e = sum of hist[s] over the slots s whose old expert is e (step 1).
    Slots holding no expert (-1) are ignored."""
    L = [0] * E
    for s, e in enumerate(np.asarray(slot_expert).tolist()):
        if e >= 0:
            L[e] += int(hist[s])
    return np.array(L, dtype=np.int64)


def replica_counts(L: np.ndarray, P_total: int, R_max: int) -> np.ndarray:
    """Step 2: greedy replica counts, compared as exact fractions."""
    E = len(L)
    c = [1] * E
    for _ in range(P_total - E):
        best = None
        for e in range(E):
            if c[e] >= R_max:
                continue
            share = Fraction(int(L[e]), c[e])
            if best is None or share > best[0]:
                best = (share, e)
        if best is None:
            raise ValueError("replica cap too small for the slot count")
        c[best[1]] += 1
    return np.array(c, dtype=np.int64)


def place(L: np.ndarray, c: np.ndarray, n_ranks: int, P_total: int):
    """Step 3: the rank of each replica.  Returns a list of (e, rank) in
    placement order."""
    per = P_total // n_ranks
    reps = [(Fraction(int(L[e]), int(c[e])), e, i) for e in range(len(L)) for i in range(int(c[e]))]
    reps.sort(key=lambda r: (-r[0], r[1], r[2]))
    load = [0.0] * n_ranks
    fill = [0] * n_ranks
    holds = [set() for _ in range(n_ranks)]
    out = []
    for _, e, _i in reps:
        best = None
        for r in range(n_ranks):
            if fill[r] == per:
                continue
            key = (e in holds[r], load[r], r)
            if best is None or key < best:
                best = key
        r = best[2]
        fill[r] += 1
        load[r] += float(L[e]) / float(c[e])
        holds[r].add(e)
        out.append((e, r))
    return out


def assign_slots(placed, slot_expert_old: np.ndarray, n_ranks: int, P_total: int) -> np.ndarray:
    """Step 4: slot of each placed replica, keeping old slots where possible."""
    per = P_total // n_ranks
    old = np.asarray(slot_expert_old).tolist()
    new = [-1] * P_total
    for r in range(n_ranks):
        slots = list(range(r * per, (r + 1) * per))
        mine = [e for e, rr in placed if rr == r]
        waiting = []
        for e in mine:
            keep = [s for s in slots if old[s] == e and new[s] < 0]
            if keep:
                new[keep[0]] = e
            else:
                waiting.append(e)
        free = [s for s in slots if new[s] < 0]
        for e, s in zip(waiting, free):
            new[s] = e
    return np.array(new, dtype=np.int32)


def rebalance(hist: np.ndarray, slot_expert_old: np.ndarray, E: int, n_ranks: int,
              R_max: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Steps 1-4.  Returns (rep_count int32 [E], rep_slots int32 [E, R_max]
    with -1 padding, slot_expert int32 [P_total])."""
    P_total = len(slot_expert_old)
    if P_total % n_ranks or P_total < E or E * R_max < P_total:
        raise ValueError("bad EPLB shape")
    L = expert_loads(hist, slot_expert_old, E)
    c = replica_counts(L, P_total, R_max)
    placed = place(L, c, n_ranks, P_total)
    slot_expert = assign_slots(placed, slot_expert_old, n_ranks, P_total)
    rep_slots = -np.ones((E, R_max), np.int32)
    rep_count = np.zeros(E, np.int32)
    for s in range(P_total):          # ascending slot order
        e = int(slot_expert[s])
        rep_slots[e, rep_count[e]] = s
        rep_count[e] += 1
    return rep_count, rep_slots, slot_expert


def migration_sources(slot_expert_old: np.ndarray, slot_expert_new: np.ndarray,
                      p0: int, P_local: int) -> np.ndarray:
    """Per local slot: the logical expert whose weights must be copied in, or
    -1 when the slot keeps its expert."""
    o = np.asarray(slot_expert_old)[p0:p0 + P_local]
    n = np.asarray(slot_expert_new)[p0:p0 + P_local]
    return np.where(o == n, -1, n).astype(np.int32)


def migrate(slots: np.ndarray, pool: np.ndarray, src: np.ndarray) -> np.ndarray:
    """Weights after migration: slot s takes pool[src[s]] when src[s] >= 0 and
    keeps its bytes otherwise.  ``slots`` [P_local, ...], ``pool`` [E, ...]."""
    out = np.array(slots, copy=True)
    for s, e in enumerate(np.asarray(src).tolist()):
        if e >= 0:
            out[s] = pool[e]
    return out


def slot_loads(hist: np.ndarray) -> Tuple[int, float]:
    """Max and mean of a per-slot load histogram (the balance EPLB improves)."""
    h = np.asarray(hist, dtype=np.int64)
    return int(h.max()), float(h.mean())
