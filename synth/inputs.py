"""Seeded synthetic workloads for one GPU's share of the fused MoE expert layer.

Every array is drawn from ``numpy.random.Generator(PCG64)`` seeded by a
``SeedSequence`` whose entropy is a tuple ``(key, stream, sub)``, so each
stream is independent of draw order and of the other streams:

* stream 0: router logits, N(0, 1) f32, row-major [T, E];
* stream 1: activations, N(0, 1) f32 rounded to bf16 (round-to-nearest-even);
* stream 2: expert weights, one seed per (logical expert, matrix), N(0, 0.02)
  f32 encoded to MXFP4 by the OCP MX v1.0 rule (the checkpoint format the
  layer consumes; see ``_encode_mxfp4``);
* stream 3: EPLB placement (the expert-popularity permutation of the skewed
  workload).

The shapes are the pages' setting: DeepSeek-V4-Pro served with EP8 on
8xMI355X, top-6 routed experts, MXFP4 routed experts with fp8 activations
("a8w4"), at most 8192 tokens per rank [sglang PR 35619 "Aiter/FlyDSL
MegaMoEv2 backend for DeepSeek-V4", reviewer reproduction and "Four settings
that silently break it"; InferenceX PR 3430, "Additional detail section";
FlyDSL issue 978, "Test environment"].  Model widths (7168 / 2048 / 384
experts) are not printed on the pages; they are the stated workload of this
repository.

Nothing here computes any part of the layer itself.  The skewed-routing bias
is fitted in closed form (a Gaussian tail condition, no top-k selection) and
the replica map is a greedy placement over the target popularity.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import os
import threading
from typing import Dict, Optional, Tuple

import numpy as np

STREAM_LOGITS = 0
STREAM_X = 1
STREAM_W = 2
STREAM_EPLB = 3

W_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Dims:
    """Problem sizes of one call (one GPU's share of one MoE layer).

    T tokens on this GPU (T_max is the capacity bucket), model width H, expert
    hidden width F, E logical experts, top-k, P_total physical expert slots
    over all ranks, of which slots [p0, p0 + P_local) live on this GPU, and
    R_max the widest replica list of the EPLB table.  ``token_id_base`` is the
    global id of token 0 (the EPLB remap hashes global token ids).
    """

    T: int
    T_max: int
    H: int
    F: int
    E: int
    k: int
    P_total: int
    p0: int
    P_local: int
    R_max: int
    token_id_base: int = 0

    def replace(self, **kw) -> "Dims":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass
class Workload:
    name: str
    dims: Dims
    logits: np.ndarray        # f32 [T, E]
    x: np.ndarray             # u16 (bf16 bit patterns) [T, H]
    rep_count: np.ndarray     # i32 [E]      replicas of each logical expert
    rep_slots: np.ndarray     # i32 [E, R_max] physical slot of each replica (-1 pad)
    slot_expert: np.ndarray   # i32 [P_local] logical expert held by each local slot
    w1: np.ndarray            # u8 [P_local, 2F, H/2]  e2m1 pairs, low nibble = even k
    w1s: np.ndarray           # u8 [P_local, 2F, H/32] e8m0 block scales
    w2: np.ndarray            # u8 [P_local, H, F/2]
    w2s: np.ndarray           # u8 [P_local, H, F/32]
    popularity: Optional[np.ndarray] = None  # target pair share per logical expert (skewed case)

    def hashes(self) -> Dict[str, str]:
        return {n: sha256(getattr(self, n)) for n in
                ("logits", "x", "rep_count", "rep_slots", "w1", "w1s", "w2", "w2s")}


# ----------------------------------------------------------------------------
# The named workloads ("key" seeds their draws):
#   tiny: T=64, H=256, F=128, E=8, top-2, all experts local
#   decode512: one EP8 rank's decode share, T=512, H=7168, F=2048, E=384,
#              top-6, 48 local experts
#   prefill8192: the prefill share, T=8192, same shapes
#   eplb8192: skewed routing + EPLB, T=8192, 448 physical slots (64
#             redundant), 56 local
#   sweep: T in {1, 8, 64, 256, 512, 1024, 4096, 8192}, decode512 shapes
# ----------------------------------------------------------------------------

WORKLOADS = {
    "tiny": dict(key=0, T=64, H=256, F=128, E=8, k=2, P_local=8, weights_key=0),
    "decode512": dict(key=1, T=512, H=7168, F=2048, E=384, k=6, P_local=48, weights_key=1),
    "prefill8192": dict(key=2, T=8192, H=7168, F=2048, E=384, k=6, P_local=48, weights_key=1),
    "eplb8192": dict(key=3, T=8192, H=7168, F=2048, E=384, k=6, P_local=56, weights_key=1,
                     redundant=64, ranks=8, zipf_s=1.2),
    "sweep": dict(key=4, T=None, H=7168, F=2048, E=384, k=6, P_local=48, weights_key=1),
}
SWEEP_T = (1, 8, 64, 256, 512, 1024, 4096, 8192)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# Input encoders (checkpoint / activation preparation, not the layer's math)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round finite f32 values to bf16 (nearest, ties to even); returns u16 bits."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _encode_mxfp4(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Encode f32 rows [R, K] to MXFP4 (OCP MX v1.0, block of 32 along K).

    Shared scale 2^X with X = floor(log2(amax)) - 2 (2 is e2m1's largest
    exponent), clamped to [-127, 127]; an all-zero block takes X = -127.
    Elements are rounded to the e2m1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} to
    nearest, ties to even, and saturate at 6.  Codes are sign-magnitude
    nibbles; element 2i sits in the low nibble of byte i.
    """
    R, K = w.shape
    b = w.reshape(R, K // 32, 32)
    amax = np.abs(b).max(axis=-1)
    _, ex = np.frexp(amax)
    X = np.where(amax > 0, ex.astype(np.int32) - 3, -127)
    X = np.clip(X, -127, 127).astype(np.int32)
    v = np.ldexp(b, (-X)[..., None]).astype(np.float32)
    a = np.abs(v)
    q = np.where(a < 2, np.rint(a * 2) * 0.5, np.where(a < 4, np.rint(a), 2 * np.rint(a * 0.5)))
    q = np.minimum(q, 6.0)
    idx = np.where(q < 2, q * 2, np.where(q < 4, q + 2, q * 0.5 + 4)).astype(np.uint8)
    sign = ((v < 0) & (q > 0)).astype(np.uint8)
    code = (idx | (sign << 3)).reshape(R, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (X + 127).astype(np.uint8).reshape(R, K // 32)
    return packed, scales


# ----------------------------------------------------------------------------
# Expert weights (cached per process: the 7168/2048 family is shared by every full-size workload)
# ----------------------------------------------------------------------------

_W_CACHE: Dict[tuple, Tuple[np.ndarray, ...]] = {}
_W_LOCK = threading.Lock()


def _expert_weights(weights_key: int, H: int, F: int, e: int,
                    std: Tuple[float, float] = (W_STD, W_STD)) -> Tuple[np.ndarray, ...]:
    ck = (weights_key, H, F, e, std)
    with _W_LOCK:
        hit = _W_CACHE.get(ck)
    if hit is not None:
        return hit
    g1 = _rng(weights_key, STREAM_W, e, 1)
    w1f = (g1.standard_normal((2 * F, H), dtype=np.float32) * np.float32(std[0]))
    w1, w1s = _encode_mxfp4(w1f)
    del w1f
    g2 = _rng(weights_key, STREAM_W, e, 2)
    w2f = (g2.standard_normal((H, F), dtype=np.float32) * np.float32(std[1]))
    w2, w2s = _encode_mxfp4(w2f)
    del w2f
    out = (w1, w1s, w2, w2s)
    with _W_LOCK:
        _W_CACHE[ck] = out
    return out


def clear_cache() -> None:
    with _W_LOCK:
        _W_CACHE.clear()


def _slot_weights(weights_key: int, H: int, F: int, slot_expert: np.ndarray,
                  std: Tuple[float, float] = (W_STD, W_STD)):
    P = len(slot_expert)
    w1 = np.empty((P, 2 * F, H // 2), np.uint8)
    w1s = np.empty((P, 2 * F, H // 32), np.uint8)
    w2 = np.empty((P, H, F // 2), np.uint8)
    w2s = np.empty((P, H, F // 32), np.uint8)
    uniq = sorted(set(int(e) for e in slot_expert))
    with _cf.ThreadPoolExecutor(_workers()) as ex:
        got = dict(zip(uniq, ex.map(lambda e: _expert_weights(weights_key, H, F, e, std), uniq)))
    for s, e in enumerate(slot_expert):
        a, b, c, d = got[int(e)]
        w1[s], w1s[s], w2[s], w2s[s] = a, b, c, d
    return w1, w1s, w2, w2s


# ----------------------------------------------------------------------------
# Tokens
# ----------------------------------------------------------------------------

def _normal_rows(key: int, stream: int, sub: int, T: int, W: int) -> np.ndarray:
    return _rng(key, stream, sub).standard_normal((T, W), dtype=np.float32)


def _tokens(key: int, sub: int, T: int, H: int, E: int, bias: Optional[np.ndarray]):
    logits = _normal_rows(key, STREAM_LOGITS, sub, T, E)
    if bias is not None:
        logits = (logits + bias.astype(np.float32)[None, :]).astype(np.float32)
    x = f32_to_bf16_bits(_normal_rows(key, STREAM_X, sub, T, H))
    return np.ascontiguousarray(logits), np.ascontiguousarray(x)


# ----------------------------------------------------------------------------
# Skewed routing (eplb8192): Zipf target popularity, closed-form bias, greedy map
# ----------------------------------------------------------------------------

def zipf_popularity(E: int, k: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Target share of (token, expert) pairs per logical expert.

    p_e proportional to rank_e^-s over a seeded permutation of the experts,
    then capped at 1/k by water-filling (a token picks an expert at most
    once, so no expert can take more than a 1/k share of the pairs).
    """
    ranks = rng.permutation(E) + 1
    p = ranks.astype(np.float64) ** (-s)
    p /= p.sum()
    cap = 1.0 / k
    fixed = np.zeros(E, bool)
    for _ in range(E):
        over = (p > cap) & ~fixed
        if not over.any():
            break
        fixed |= over
        p[fixed] = cap
        rest = ~fixed
        p[rest] *= (1.0 - cap * fixed.sum()) / p[rest].sum()
    return p


def zipf_bias(p: np.ndarray, k: int) -> np.ndarray:
    """Per-expert logit bias giving pair shares close to ``p``.

    With logits b_e + N(0, 1), a mean-field threshold at 0 puts expert e in a
    token's top-k with probability Phi(b_e); asking Phi(b_e) = k p_e (which
    sums to k over the experts) gives b_e = Phi^-1(k p_e).  The achieved
    shares are measured, not assumed.
    """
    from scipy.special import ndtri
    q = np.clip(k * p, 1e-9, 1.0 - 1e-6)
    return ndtri(q).astype(np.float32)


def greedy_replica_map(p: np.ndarray, redundant: int, ranks: int):
    """Seeded greedy EPLB placement.

    1. every expert starts with one replica; ``redundant`` times, add a replica
       to argmax_e p_e / c_e (ties to the lower e);
    2. order the replicas by p_e / c_e descending (ties by e, then replica);
    3. put each on the least-loaded rank that has a free slot, preferring
       ranks without a copy of e (ties to the lower rank);
    4. slot id = rank * slots_per_rank + fill order.
    Returns (rep_count [E], rep_slots [E, R_max] (-1 pad), slot_expert [P_total]).
    """
    E = len(p)
    c = np.ones(E, np.int64)
    for _ in range(redundant):
        c[int(np.argmax(p / c))] += 1
    P_total = E + redundant
    assert P_total % ranks == 0
    per = P_total // ranks
    reps = [(p[e] / c[e], e, i) for e in range(E) for i in range(int(c[e]))]
    reps.sort(key=lambda r: (-r[0], r[1], r[2]))
    load = np.zeros(ranks)
    fill = np.zeros(ranks, np.int64)
    holds = [set() for _ in range(ranks)]
    R_max = int(c.max())
    rep_slots = -np.ones((E, R_max), np.int32)
    nrep = np.zeros(E, np.int64)
    slot_expert = -np.ones(P_total, np.int32)
    for share, e, _ in reps:
        best = None
        for r in range(ranks):
            if fill[r] >= per:
                continue
            key = (e in holds[r], load[r], r)
            if best is None or key < best[0]:
                best = (key, r)
        r = best[1]
        slot = r * per + int(fill[r])
        fill[r] += 1
        load[r] += share
        holds[r].add(e)
        rep_slots[e, nrep[e]] = slot
        nrep[e] += 1
        slot_expert[slot] = e
    return c.astype(np.int32), rep_slots, slot_expert


def naive_replica_map(E: int, P_total: int):
    """Naive placement (no load information): slot s holds logical expert
    s mod E, so the P_total - E redundant slots copy experts 0, 1, ... in
    order.  Returns (rep_count [E], rep_slots [E, R_max] (-1 pad),
    slot_expert [P_total]); each expert's slots in ascending order."""
    slot_expert = (np.arange(P_total) % E).astype(np.int32)
    rep_count = np.bincount(slot_expert, minlength=E).astype(np.int32)
    R_max = int(rep_count.max())
    rep_slots = -np.ones((E, R_max), np.int32)
    fill = np.zeros(E, np.int64)
    for s, e in enumerate(slot_expert.tolist()):
        rep_slots[e, fill[e]] = s
        fill[e] += 1
    return rep_count, rep_slots, slot_expert


def skewed_logits(key: int, sub: int, T: int, E: int, k: int, s: float = 1.2) -> np.ndarray:
    """Router logits whose expert popularity follows Zipf(s) (capped at 1/k):
    N(0, 1) plus the per-expert bias of ``zipf_bias``."""
    pop = zipf_popularity(E, k, s, _rng(key, STREAM_EPLB, 0))
    return _tokens(key, sub, T, 128, E, zipf_bias(pop, k))[0]


def expert_weights(weights_key: int, H: int, F: int, experts,
                   w_std: Tuple[float, float] = (W_STD, W_STD)):
    """Natural MXFP4 weights of the listed logical experts, stacked in list
    order: (w1 [n, 2F, H/2], w1s [n, 2F, H/32], w2 [n, H, F/2], w2s [n, H, F/32])."""
    return _slot_weights(weights_key, H, F, np.asarray(list(experts), np.int32), tuple(w_std))


def token_batch(key: int, sub: int, T: int, H: int, E: int, k: int, zipf_s: Optional[float] = None):
    """One batch of router logits (f32 [T, E], Zipf-skewed if ``zipf_s``) and
    activations (bf16 bits [T, H]); ``sub`` picks an independent draw."""
    bias = None
    if zipf_s is not None:
        bias = zipf_bias(zipf_popularity(E, k, zipf_s, _rng(key, STREAM_EPLB, 0)), k)
    return _tokens(key, sub, T, H, E, bias)


def with_replica_map(wl: "Workload", rep_count, rep_slots, slot_expert_all, p0: int, P_local: int,
                     weights_key: int, w_std: Tuple[float, float] = (W_STD, W_STD),
                     logits: Optional[np.ndarray] = None, x: Optional[np.ndarray] = None,
                     token_id_base: Optional[int] = None) -> "Workload":
    """``wl`` with another replica table: slots [p0, p0 + P_local) of
    ``slot_expert_all`` on this GPU, their weights drawn with ``weights_key``;
    optionally another token batch."""
    slot_expert_all = np.asarray(slot_expert_all, np.int32)
    rep_slots = np.asarray(rep_slots, np.int32)
    lg = wl.logits if logits is None else logits
    xx = wl.x if x is None else x
    base = wl.dims.token_id_base if token_id_base is None else token_id_base
    d = wl.dims.replace(T=lg.shape[0], T_max=max(wl.dims.T_max, lg.shape[0]), P_total=len(slot_expert_all),
                        p0=p0, P_local=P_local, R_max=rep_slots.shape[1], token_id_base=base)
    se = slot_expert_all[p0:p0 + P_local].copy()
    w1, w1s, w2, w2s = _slot_weights(weights_key, d.H, d.F, se, tuple(w_std))
    return Workload(name=wl.name + f"_map{len(slot_expert_all)}", dims=d, logits=lg, x=xx,
                    rep_count=np.asarray(rep_count, np.int32), rep_slots=rep_slots, slot_expert=se,
                    w1=w1, w1s=w1s, w2=w2, w2s=w2s, popularity=wl.popularity)


STREAM_GATE = 5


def gate_weights(key: int, E: int, H: int) -> np.ndarray:
    """Router gate weights W_gate [E, H] as bf16 bits: N(0, 1/H) rounded to
    bf16, so that the logits of N(0, 1) activations are close to N(0, 1) (the
    logits the layer's workloads draw directly)."""
    g = _rng(key, STREAM_GATE, 0)
    return f32_to_bf16_bits(g.standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H)))


# ----------------------------------------------------------------------------
# Public constructors
# ----------------------------------------------------------------------------

def dims_for(name: str, T: Optional[int] = None, T_max: Optional[int] = None) -> Dims:
    c = WORKLOADS[name]
    T = c["T"] if T is None else T
    E, k = c["E"], c["k"]
    if c.get("redundant"):
        P_total = E + c["redundant"]
        R_max = None  # fixed after the map is built
    else:
        P_total, R_max = E, 1
    return Dims(T=T, T_max=T if T_max is None else T_max, H=c["H"], F=c["F"], E=E, k=k,
                P_total=P_total, p0=0, P_local=c["P_local"], R_max=R_max or 1)


def _identity_map(E: int):
    return np.ones(E, np.int32), np.arange(E, dtype=np.int32)[:, None].copy()


def make(name: str, T: Optional[int] = None, with_weights: bool = True,
         sub: int = 0, token_id_base: int = 0, p0: int = 0) -> Workload:
    """Workload ``name`` (a key of WORKLOADS).  ``T`` overrides the token count
    (required for "sweep").

    ``sub`` selects an independent token draw (the virtual rank of the
    EP-shaped prefill case, or the T point of the sweep); ``p0`` moves this
    GPU's window of physical slots.
    """
    c = WORKLOADS[name]
    key = c["key"]
    if c["T"] is None:
        if T is None:
            raise ValueError(f"workload {name} needs T")
        sub = T if sub == 0 else sub
    d = dims_for(name, T)
    E, H, F, k = d.E, d.H, d.F, d.k
    bias = None
    pop = None
    if c.get("redundant"):
        g = _rng(key, STREAM_EPLB, 0)
        pop = zipf_popularity(E, k, c["zipf_s"], g)
        bias = zipf_bias(pop, k)
        rep_count, rep_slots, all_slot_expert = greedy_replica_map(pop, c["redundant"], c["ranks"])
        d = d.replace(R_max=rep_slots.shape[1])
    else:
        rep_count, rep_slots = _identity_map(E)
        all_slot_expert = np.arange(E, dtype=np.int32)
    d = d.replace(p0=p0, token_id_base=token_id_base)
    if p0 < 0 or p0 + d.P_local > d.P_total:
        raise ValueError("local slot window out of range")
    slot_expert = all_slot_expert[p0:p0 + d.P_local].copy()
    logits, x = _tokens(key, sub, d.T, H, E, bias)
    if with_weights:
        w1, w1s, w2, w2s = _slot_weights(c["weights_key"], H, F, slot_expert)
    else:
        z = np.zeros((0,), np.uint8)
        w1 = w1s = w2 = w2s = z
    return Workload(name=name + (f"_T{d.T}" if c["T"] is None else ""), dims=d,
                    logits=logits, x=x, rep_count=rep_count, rep_slots=rep_slots,
                    slot_expert=slot_expert, w1=w1, w1s=w1s, w2=w2, w2s=w2s,
                    popularity=pop)


def make_sweep(T: int, with_weights: bool = True) -> Workload:
    return make("sweep", T=T, with_weights=with_weights)


def make_ep_shaped(ranks: int = 8, T_rank: int = 8192, with_weights: bool = True) -> Workload:
    """The prefill share at a real EP rank's load.

    ``ranks`` virtual ranks of ``T_rank`` tokens each (rank r's tokens are the
    prefill8192 draw with sub = r, global ids r*T_rank + t) all route into this
    GPU's 48 experts, as every rank's tokens do under EP8.
    """
    parts = [make("prefill8192", with_weights=False, sub=r) for r in range(ranks)]
    base = parts[0]
    logits = np.concatenate([p.logits for p in parts])
    x = np.concatenate([p.x for p in parts])
    T = ranks * T_rank
    d = base.dims.replace(T=T, T_max=T)
    w = make("prefill8192", T=1, with_weights=with_weights) if with_weights else base
    return Workload(name=f"prefill8192_ep{ranks}", dims=d, logits=logits, x=x,
                    rep_count=base.rep_count, rep_slots=base.rep_slots,
                    slot_expert=base.slot_expert, w1=w.w1, w1s=w.w1s, w2=w.w2, w2s=w.w2s)


def make_custom(T: int, H: int, F: int, E: int, k: int, P_local: int, p0: int = 0,
                redundant: int = 0, ranks: int = 1, seed: int = 100, token_id_base: int = 0,
                T_max: Optional[int] = None, zipf_s: Optional[float] = None,
                w_std: Tuple[float, float] = (W_STD, W_STD)) -> Workload:
    """A workload of arbitrary shape (parity cases that span several tiles and
    ragged tails).  ``redundant`` > 0 adds replicas by the greedy map over a
    uniform (or Zipf, if ``zipf_s``) popularity; physical slots are spread over
    ``ranks`` ranks and this GPU holds [p0, p0 + P_local).  ``w_std``: the
    standard deviations of W1 and W2 (both 0.02 by default)."""
    pop = None
    bias = None
    if zipf_s is not None:
        pop = zipf_popularity(E, k, zipf_s, _rng(seed, STREAM_EPLB, 0))
        bias = zipf_bias(pop, k)
    if redundant > 0:
        p = pop if pop is not None else np.full(E, 1.0 / E)
        rep_count, rep_slots, all_slot_expert = greedy_replica_map(p, redundant, ranks)
    else:
        rep_count, rep_slots = _identity_map(E)
        all_slot_expert = np.arange(E, dtype=np.int32)
    P_total = E + redundant
    d = Dims(T=T, T_max=T if T_max is None else T_max, H=H, F=F, E=E, k=k, P_total=P_total, p0=p0,
             P_local=P_local, R_max=rep_slots.shape[1], token_id_base=token_id_base)
    if p0 < 0 or p0 + P_local > P_total:
        raise ValueError("local slot window out of range")
    slot_expert = all_slot_expert[p0:p0 + P_local].copy()
    logits, x = _tokens(seed, 0, T, H, E, bias)
    w1, w1s, w2, w2s = _slot_weights(1000 + seed, H, F, slot_expert, tuple(w_std))
    return Workload(name=f"custom_T{T}_H{H}_F{F}_E{E}_k{k}", dims=d, logits=logits, x=x,
                    rep_count=rep_count, rep_slots=rep_slots, slot_expert=slot_expert,
                    w1=w1, w1s=w1s, w2=w2, w2s=w2s, popularity=pop)
