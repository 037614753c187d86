"""Pins of the oracle's routing, EPLB remap/record and bucketing."""

import itertools
import math
import os

import numpy as np
import torch

from oracle import moe as om
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- O1 route

def test_route_brute_force_subsets():
    rng = np.random.default_rng(0)
    T, E, k = 16, 8, 2
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = om.route(lg, k)
    for t in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(float(lg[t, e]) for e in c))
        assert set(ids[t].tolist()) == set(best)
        assert lg[t, ids[t, 0]] > lg[t, ids[t, 1]]           # descending order
        s = [1.0 / (1.0 + math.exp(-float(lg[t, e]))) for e in ids[t]]
        assert np.allclose(w[t], np.array(s) / sum(s), rtol=0, atol=1e-15)


def test_route_matches_torch_topk_and_sigmoid():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((256, 384)).astype(np.float32)
    ids, w = om.route(lg, 6)
    tv, ti = torch.topk(torch.from_numpy(lg), 6, dim=1, largest=True, sorted=True)
    assert np.array_equal(ids, ti.numpy())
    s = torch.sigmoid(tv.double())
    assert np.allclose(w, (s / s.sum(1, keepdim=True)).numpy(), rtol=1e-14, atol=0)


def test_route_ties_go_to_lower_id():
    lg = np.zeros((3, 8), np.float32)
    lg[1, [2, 5, 6]] = 1.0
    lg[2] = [0.5, 2.0, 0.5, 2.0, -1, 2.0, 0, 0]
    ids, w = om.route(lg, 3)
    assert ids[0].tolist() == [0, 1, 2]
    assert ids[1].tolist() == [2, 5, 6]
    assert ids[2].tolist() == [1, 3, 5]
    assert np.all(w == 1.0 / 3)


def test_route_special_cases():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((32, 8)).astype(np.float32)
    ids1, w1 = om.route(lg, 1)
    assert np.all(w1 == 1.0)
    assert np.array_equal(ids1[:, 0], lg.argmax(1))
    idsE, wE = om.route(lg, 8)
    assert np.all(np.sort(idsE, 1) == np.arange(8))
    assert np.allclose(wE.sum(1), 1.0, atol=1e-15)
    # sigmoid(l) + sigmoid(-l) = 1: with two chosen logits l and -l the
    # weights are exactly the two scores
    lg2 = np.full((1, 4), -9.0, np.float32)
    lg2[0, 1], lg2[0, 3] = 0.75, -0.75
    ids2, w2 = om.route(lg2, 2)
    assert ids2[0].tolist() == [1, 3]
    assert abs(w2[0, 0] - 1.0 / (1.0 + math.exp(-0.75))) < 1e-15
    assert abs(w2[0, 0] + w2[0, 1] - 1.0) < 1e-15


def test_sigmoid_stable_tails():
    z = np.array([-800.0, -40.0, 0.0, 40.0, 800.0])
    s = om.sigmoid(z)
    assert s[0] == 0.0 and s[2] == 0.5 and s[4] == 1.0
    assert abs(s[1] - math.exp(-40) / (1 + math.exp(-40))) < 1e-30


# ---------------------------------------------------------------- O2 remap + record

def _murmur3_x86_32(key: bytes, seed: int) -> int:
    """MurmurHash3_x86_32 with the oracle's fmix32 as its final step."""
    def rotl(x, r):
        return ((x << r) | (x >> (32 - r))) & 0xFFFFFFFF
    c1, c2 = 0xCC9E2D51, 0x1B873593
    h = seed
    nb = len(key) // 4
    for i in range(nb):
        k = int.from_bytes(key[4 * i:4 * i + 4], "little")
        k = rotl((k * c1) & 0xFFFFFFFF, 15)
        h ^= (k * c2) & 0xFFFFFFFF
        h = (rotl(h, 13) * 5 + 0xE6546B64) & 0xFFFFFFFF
    tail = key[4 * nb:]
    k = 0
    for i in reversed(range(len(tail))):
        k ^= tail[i] << (8 * i)
    if tail:
        k = rotl((k * c1) & 0xFFFFFFFF, 15)
        h ^= (k * c2) & 0xFFFFFFFF
    h ^= len(key)
    return int(om.fmix32(np.array([h], np.uint32))[0])


def test_fmix32_published_murmur3_vectors():
    with open(os.path.join(GOLD, "murmur3_x86_32.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) >= 7
    for key_hex, seed, want in rows:
        key = b"" if key_hex == "-" else bytes.fromhex(key_hex)
        assert _murmur3_x86_32(key, int(seed, 16)) == int(want, 16), key_hex


def test_fmix32_is_a_bijection():
    """Invert each step (xor-shift and odd multiply) and recover the input."""
    rng = np.random.default_rng(3)
    x = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64)
    h = om.fmix32(x).astype(np.uint64)

    def unxorshift(v, s):
        r = v.copy()
        for _ in range(32 // s + 1):
            r = v ^ (r >> s)
        return r

    inv1 = pow(0x85EBCA6B, -1, 2 ** 32)
    inv2 = pow(0xC2B2AE35, -1, 2 ** 32)
    v = unxorshift(h, 16)
    v = (v * inv2) & 0xFFFFFFFF
    v = unxorshift(v, 13)
    v = (v * inv1) & 0xFFFFFFFF
    v = unxorshift(v, 16)
    assert np.array_equal(v, x)
    assert om.fmix32(np.array([0], np.uint32))[0] == 0


def test_remap_identity_and_histogram_brute_force():
    rng = np.random.default_rng(4)
    T, E, k = 40, 16, 3
    ids, _ = om.route(rng.standard_normal((T, E)).astype(np.float32), k)
    rc = np.ones(E, np.int32)
    rs = np.arange(E, dtype=np.int32)[:, None]
    phys, hist = om.remap_record(ids, rc, rs, 1234, E)
    assert np.array_equal(phys, ids)
    brute = [0] * E
    for t in range(T):
        for j in range(k):
            brute[int(phys[t, j])] += 1
    assert hist.tolist() == brute and hist.sum() == T * k


def test_remap_replicas_follow_the_hash():
    E, T, k = 4, 64, 2
    rc = np.array([1, 2, 3, 1], np.int32)
    rs = np.array([[0, -1, -1], [1, 4, -1], [2, 5, 6], [3, -1, -1]], np.int32)
    ids = np.tile(np.array([[1, 2]], np.int32), (T, 1))
    base = 1000
    phys, hist = om.remap_record(ids, rc, rs, base, 7)
    for t in range(T):
        h = _murmur3_x86_32(b"", base + t)  # empty key: fmix32(seed)
        assert phys[t, 0] == rs[1, h % 2]
        assert phys[t, 1] == rs[2, h % 3]
    assert hist[[1, 4]].sum() == T and hist[[2, 5, 6]].sum() == T
    assert hist[0] == hist[3] == 0
    # every replica gets used, none outside the table
    assert min(hist[[1, 4, 2, 5, 6]]) > 0


def test_remap_token_id_wraps_mod_2_32():
    ids = np.zeros((2, 1), np.int32)
    rc = np.array([5], np.int32)
    rs = np.arange(5, dtype=np.int32)[None, :]
    phys, _ = om.remap_record(ids, rc, rs, 2 ** 32 - 1, 5)
    assert phys[0, 0] == _murmur3_x86_32(b"", 2 ** 32 - 1) % 5
    assert phys[1, 0] == 0   # fmix32(0) = 0


# ---------------------------------------------------------------- O3 buckets

def test_buckets_against_python_loops():
    rng = np.random.default_rng(5)
    T, k, P_total = 50, 3, 20
    phys = rng.integers(0, P_total, size=(T, k)).astype(np.int32)
    p0, PL = 6, 8
    counts, offsets, rop, por = om.buckets(phys, p0, PL)
    rows = {}
    for t in range(T):
        for j in range(k):
            p = int(phys[t, j])
            if p0 <= p < p0 + PL:
                rows.setdefault(p - p0, []).append(t * k + j)
    assert counts.tolist() == [len(rows.get(s, [])) for s in range(PL)]
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    for s in range(PL):
        assert por[offsets[s]:offsets[s + 1]].tolist() == rows.get(s, [])
    for p in range(T * k):
        if rop[p] >= 0:
            assert por[rop[p]] == p
        else:
            assert not (p0 <= phys.ravel()[p] < p0 + PL)
    assert (rop >= 0).sum() == offsets[-1]


def test_buckets_empty_and_all_remote():
    phys = np.full((5, 2), 30, np.int32)
    counts, offsets, rop, por = om.buckets(phys, 0, 8)
    assert counts.sum() == 0 and offsets.tolist() == [0] * 9 and np.all(rop == -1) and por.size == 0
    counts, offsets, rop, por = om.buckets(np.zeros((0, 2), np.int32), 0, 8)
    assert counts.sum() == 0 and rop.size == 0


# ---------------------------------------------------------------- input tables

def test_greedy_replica_map_is_a_valid_placement():
    wl = synth.make("eplb8192", T=16, with_weights=False)
    d = wl.dims
    assert d.P_total == 448 and d.P_local == 56
    rc, rs = wl.rep_count, wl.rep_slots
    assert rc.sum() == 448 and rc.min() >= 1
    used = rs[rs >= 0]
    assert np.array_equal(np.sort(used), np.arange(448))       # each slot exactly once
    for e in range(d.E):
        assert (rs[e] >= 0).sum() == rc[e]
    # popular experts got the replicas
    pop = wl.popularity
    assert rc[np.argmax(pop)] == rc.max()
    assert abs(pop.sum() - 1) < 1e-12 and pop.max() <= 1.0 / 6 + 1e-12


def test_skewed_routing_is_skewed_and_map_balances_it():
    wl = synth.make("eplb8192", T=2048, with_weights=False)
    d = wl.dims
    ids, _ = om.route(wl.logits, d.k)
    share = np.bincount(ids.ravel(), minlength=d.E) / ids.size
    order = np.argsort(-wl.popularity)
    top = share[order[:8]].sum()
    assert top > 0.25                                         # Zipf head takes a large share
    phys, hist = om.remap_record(ids, wl.rep_count, wl.rep_slots, 0, d.P_total)
    per_rank = hist.reshape(8, 56).sum(1)
    logical_rank = np.bincount(ids.ravel() // 48, minlength=8)
    assert per_rank.max() / per_rank.mean() < logical_rank.max() / logical_rank.mean()
