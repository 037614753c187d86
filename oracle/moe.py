"""Plain, slow, float64 CPU oracle of one GPU's share of the fused MoE expert layer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

What the layer computes, per the pages: the MegaMoEV2 operator runs quant,
dispatch, GEMM1, GEMM2 and combine for the routed experts [sglang PR 47065
"[Perf] [AMD] dsv4: Use the aiter MegaMoE small- and large-input paths",
intro], with fp8 activations on MXFP4 experts ("a8w4") [InferenceX PR 3430
"[AMD][MI35X] 0926 DSV4 sglang mtp agentic", Additional detail section], top-6
routing [sglang PR 35619 "Aiter/FlyDSL MegaMoEv2 backend for DeepSeek-V4",
"Four settings that silently break it", item 2], and, in prefill, a fused
EPLB logical-to-physical remap with load recording [same page, Summary;
FlyDSL issue 978, Benchmark plan and Data-quality gates].  The pages give no
formula for any step.  Where they are silent this module takes the readings
listed with each function (sigmoid scores, renormalised weights, SwiGLU,
e8m0 per-128 activation scales, a MurmurHash3 finaliser as the token hash).

Stages (numbers match the hot-path table of the design notes):
  O1 route      O2 remap + record      O3 buckets
  O4 act quant  O5 GEMM1  O6 SwiGLU    O7 requant
  O8 GEMM2      O9 combine
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import formats as fm

BLOCK_ACT = 128  # activation scale block (columns)


# ----------------------------------------------------------------------------
# O1 route
# ----------------------------------------------------------------------------

def sigmoid(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def route(logits: np.ndarray, k: int):
    """Top-k experts per token and their routing weights.

    Reading (the pages name top-6 routing only): scores are sigmoid(logit);
    the k experts with the largest logits are selected (sigmoid is strictly
    increasing, so this is top-k on the scores without the ties that rounding
    a sigmoid would create), in descending order, equal logits going to the
    lower expert id; weights are the selected scores divided by their sum.
    Returns ids int32 [T, k] and weights float64 [T, k].
    """
    lg = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    s = sigmoid(np.take_along_axis(lg, ids, axis=1).astype(np.float64))
    w = s / s.sum(axis=1, keepdims=True)
    return ids, w


# ----------------------------------------------------------------------------
# O2 EPLB remap + record
# ----------------------------------------------------------------------------

def fmix32(h) -> np.ndarray:
    """MurmurHash3's 32-bit finaliser (Appleby, public domain):
    xor-shift 16, multiply 0x85ebca6b, xor-shift 13, multiply 0xc2b2ae35,
    xor-shift 16, all modulo 2^32."""
    h = np.asarray(h, dtype=np.uint64) & 0xFFFFFFFF
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & 0xFFFFFFFF
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & 0xFFFFFFFF
    h ^= h >> 16
    return h.astype(np.uint32)


def remap_record(ids: np.ndarray, rep_count: np.ndarray, rep_slots: np.ndarray,
                 token_id_base: int, P_total: int):
    """Logical -> physical expert, and the per-physical-slot load histogram.

    Reading: token t's pairs go to replica fmix32(token_id_base + t) mod
    rep_count[e] of their logical expert e; the histogram counts every
    (token, expert) pair of this GPU's tokens over all P_total slots (the
    recorder's "stat" mode counts load per physical expert).  Returns
    phys int32 [T, k] and hist int64 [P_total].
    """
    T, k = ids.shape
    tok = (np.uint64(token_id_base) + np.arange(T, dtype=np.uint64)) & 0xFFFFFFFF
    h = fmix32(tok).astype(np.int64)
    cnt = rep_count[ids].astype(np.int64)
    r = h[:, None] % cnt
    phys = rep_slots[ids, r].astype(np.int32)
    hist = np.bincount(phys.ravel(), minlength=P_total)
    return phys, hist


# ----------------------------------------------------------------------------
# O3 buckets
# ----------------------------------------------------------------------------

def buckets(phys: np.ndarray, p0: int, P_local: int):
    """Group this GPU's pairs by local slot.

    A pair (t, j) is local when p0 <= phys < p0 + P_local; its local slot is
    phys - p0.  Rows of a slot are contiguous, slots in ascending order, and
    inside a slot rows follow ascending (t, j).  Returns counts [P_local],
    offsets [P_local + 1], row_of_pair [T*k] (-1 for remote pairs) and
    pair_of_row [rows] (pair index t*k + j).
    """
    flat = phys.ravel().astype(np.int64)
    local = (flat >= p0) & (flat < p0 + P_local)
    slot = np.where(local, flat - p0, -1)
    counts = np.bincount(slot[local], minlength=P_local).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_of_pair = -np.ones(flat.size, np.int64)
    nxt = offsets[:-1].copy()
    for p in range(flat.size):          # (t, j) ascending
        s = slot[p]
        if s >= 0:
            row_of_pair[p] = nxt[s]
            nxt[s] += 1
    pair_of_row = np.empty(int(offsets[-1]), np.int64)
    pair_of_row[row_of_pair[local]] = np.nonzero(local)[0]
    return counts, offsets, row_of_pair, pair_of_row


# ----------------------------------------------------------------------------
# O4 / O7 block quantisation to fp8 with e8m0 scales
# ----------------------------------------------------------------------------

def scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0), clamped to [-127, 127].

    With amax = f * 2^x, f in [0.5, 1): 448 = 0.875 * 2^9, so e = x - 9 when
    f <= 0.875 and x - 8 otherwise (x - 10 would need f <= 0.4375).
    """
    a = np.asarray(amax, dtype=np.float64)
    f, x = np.frexp(a)
    e = x.astype(np.int64) - 9 + (f > 0.875)
    e = np.where(a > 0, e, 0)
    return np.clip(e, -127, 127)


def quant_blocks(v: np.ndarray, block: int = BLOCK_ACT):
    """Quantise rows [N, W] (float64) per block of ``block`` columns.

    Reading of "per-token per-128-column scales": the scale is an e8m0 power
    of two 2^e, e the smallest integer with block amax <= 448 * 2^e; every
    element becomes RNE_e4m3fn(v * 2^-e), an exact scaling followed by one
    rounding.  Returns codes u8 [N, W] and scale bytes u8 [N, W/block]
    (byte = e + 127).
    """
    v = np.asarray(v, dtype=np.float64)
    N, W = v.shape
    b = v.reshape(N, W // block, block)
    e = scale_exponent(np.abs(b).max(axis=-1))
    scaled = np.ldexp(b, (-e)[..., None])
    q = fm.enc_e4m3fn_rne(scaled).reshape(N, W)
    return q, (e + 127).astype(np.uint8)


def dequant_blocks(q: np.ndarray, s: np.ndarray, block: int = BLOCK_ACT) -> np.ndarray:
    vals = fm.dec_e4m3fn(q)
    return vals * np.repeat(fm.dec_e8m0(s), block, axis=-1)


# ----------------------------------------------------------------------------
# O5-O8 one expert
# ----------------------------------------------------------------------------

def silu(g) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g)


def gemm1_swiglu(a: np.ndarray, w1: np.ndarray, w1s: np.ndarray, F: int):
    """h = a W1^T (float64), W1 rows [0, F) gate and [F, 2F) up; act = silu(gate) * up.

    Reading (the pages only say GEMM1 then GEMM2): SwiGLU, no clamp, float64.
    Returns (act [n, F], h [n, 2F]).
    """
    W = fm.dequant_mxfp4(w1, w1s)
    h = a @ W.T
    return silu(h[:, :F]) * h[:, F:], h


def gemm2(act_dq: np.ndarray, w2: np.ndarray, w2s: np.ndarray) -> np.ndarray:
    """y = act W2^T in float64."""
    return act_dq @ fm.dequant_mxfp4(w2, w2s).T


def expert_rows(xq_rows, xs_rows, w1, w1s, w2, w2s, F: int):
    """O5-O8 for the rows of one local slot.  Returns dict act, h, aq, as_, y."""
    a = dequant_blocks(xq_rows, xs_rows)
    act, h = gemm1_swiglu(a, w1, w1s, F)
    aq, as_ = quant_blocks(act)
    y = gemm2(dequant_blocks(aq, as_), w2, w2s)
    return dict(act=act, h=h, aq=aq, as_=as_, y=y)


# ----------------------------------------------------------------------------
# O9 combine
# ----------------------------------------------------------------------------

def combine(y: np.ndarray, row_of_pair: np.ndarray, w: np.ndarray, T: int, k: int,
            H: int) -> np.ndarray:
    """out[t] = sum over local pairs j (ascending) of w[t, j] * y[row(t, j)], in float64.

    Reading: the routing weight is applied here, after GEMM2, never before the
    requant.  Tokens with no local pair get +0.  Returns float64 [T, H].
    """
    rop = row_of_pair.reshape(T, k)
    out = np.zeros((T, H))
    for j in range(k):
        m = rop[:, j] >= 0
        if m.any():
            out[m] += w[m, j][:, None] * y[rop[m, j]]
    return out


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

def forward(wl, slots: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """All stages of the layer for a ``synth.Workload``.

    ``slots`` (optional) restricts O5-O8 to those local slots (the combine
    then sums only their pairs); used to time a bounded sample.
    Returns a dict with every intermediate and ``out_bf16`` (u16 [T, H]).
    """
    d = wl.dims
    T, H, F, k = d.T, d.H, d.F, d.k
    ids, w = route(wl.logits, k)
    phys, hist = remap_record(ids, wl.rep_count, wl.rep_slots, d.token_id_base, d.P_total)
    counts, offsets, row_of_pair, pair_of_row = buckets(phys, d.p0, d.P_local)
    rows = int(offsets[-1])
    xv = fm.bf16_to_f64(wl.x)
    xq_t, xs_t = quant_blocks(xv)                     # per token
    tok_of_row = pair_of_row // k
    xq = xq_t[tok_of_row]
    xs = xs_t[tok_of_row]
    act = np.zeros((rows, F))
    aq = np.zeros((rows, F), np.uint8)
    as_ = np.zeros((rows, F // BLOCK_ACT), np.uint8)
    y = np.zeros((rows, H))
    todo = range(d.P_local) if slots is None else slots
    done_rows = np.zeros(rows, bool)
    for s in todo:
        lo, hi = int(offsets[s]), int(offsets[s + 1])
        if hi == lo:
            continue
        r = expert_rows(xq[lo:hi], xs[lo:hi], wl.w1[s], wl.w1s[s], wl.w2[s], wl.w2s[s], F)
        act[lo:hi], aq[lo:hi], as_[lo:hi], y[lo:hi] = r["act"], r["aq"], r["as_"], r["y"]
        done_rows[lo:hi] = True
    rop = row_of_pair.copy()
    if slots is not None:
        rop[(rop >= 0) & ~done_rows[np.maximum(rop, 0)]] = -1
    out = combine(y, rop, w, T, k, H)
    return dict(topk_ids=ids, topk_w=w, phys_ids=phys, load_hist=hist, counts=counts,
                offsets=offsets, row_of_pair=row_of_pair, pair_of_row=pair_of_row,
                xq_tok=xq_t, xs_tok=xs_t, xq=xq, xs=xs, act=act, aq=aq, as_=as_, y=y,
                out=out, out_bf16=fm.f64_to_bf16_rne(out))


def forward_token(wl, t: int, ids=None, w=None, phys=None) -> np.ndarray:
    """Output row of one token computed on its own, with no bucketing.

    out[t] = sum over its local pairs of w_tj * expert_phys(x_t), each expert
    applied to the single token.  Used to check sampled tokens of the full-size
    workloads and as a second formulation of the bucketed path.
    """
    d = wl.dims
    if ids is None:
        ids, w = route(wl.logits[t:t + 1], d.k)
        phys, _ = remap_record(ids, wl.rep_count, wl.rep_slots, d.token_id_base + t, d.P_total)
        ids, w, phys = ids[0], w[0], phys[0]
    q, s = quant_blocks(fm.bf16_to_f64(wl.x[t:t + 1]))
    out = np.zeros(d.H)
    for j in range(d.k):
        p = int(phys[j])
        if not (d.p0 <= p < d.p0 + d.P_local):
            continue
        sl = p - d.p0
        r = expert_rows(q, s, wl.w1[sl], wl.w1s[sl], wl.w2[sl], wl.w2s[sl], d.F)
        out += w[j] * r["y"][0]
    return out


# ----------------------------------------------------------------------------
# Parity protocol helpers (fp8 requant of f32-vs-f64 values)
# ----------------------------------------------------------------------------

def requant_tie_zone(act: np.ndarray, eps: np.ndarray, block: int = BLOCK_ACT):
    """Where a correct float32 implementation may legitimately pick another code.

    ``eps`` bounds |act_gpu - act| elementwise.  An element is flagged when a
    rounding midpoint of the fp8 grid lies within eps * 2^-e of its scaled
    value; a block is flagged when a scale boundary 448 * 2^j lies within
    max(eps) of its amax.  Returns (elem_flags [N, W] bool, block_flags [N, W/block] bool).
    """
    N, W = act.shape
    b = act.reshape(N, W // block, block)
    eb = eps.reshape(N, W // block, block)
    amax = np.abs(b).max(axis=-1)
    e = scale_exponent(amax)
    sc = np.ldexp(np.abs(b), (-e)[..., None])
    tol = np.ldexp(eb, (-e)[..., None])
    # fp8 grid spacing at |sc|: 2^-9 below 2^-6, else 2^(floor(log2 sc) - 3)
    f, x = np.frexp(np.where(sc > 0, sc, 1.0))
    ulp = np.where(sc < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, x.astype(np.int64) - 1 - 3))
    pos = sc / ulp
    frac = pos - np.floor(pos)
    elem = np.abs(frac - 0.5) * ulp <= tol
    # an element near a binade edge can fall to the grid below, whose spacing is half
    lo_ulp = ulp / 2
    edge = (sc >= 2.0 ** -6) & (np.abs(sc - np.ldexp(1.0, x.astype(np.int64) - 1)) <= tol + lo_ulp / 2)
    elem |= edge
    bound_hi = np.ldexp(448.0, e)
    bound_lo = np.ldexp(448.0, e - 1)
    m = eb.max(axis=-1)
    blk = (np.abs(amax - bound_hi) <= m) | (np.abs(amax - bound_lo) <= m)
    return elem.reshape(N, W), blk


#: Error allowance of one block-scaled MFMA instruction (K = 128 products
#: summed inside the instruction), as a fraction of the sum of the absolute
#: values of its products, for operands distributed like the layer's.
#: Measured on gfx950 (tests/test_gpu_mfma_rounding.py): inside each 32-element
#: scale block the instruction drops the bits of its products more than about
#: 14 below the block's largest product, and combines the blocks at float32
#: precision.  On the layer's operands (N(0, 1) token rows quantised per 128
#: columns, SwiGLU-shaped act rows, N(0, 0.02) MXFP4 weights) one instruction
#: errs by at most 8.7e-6 (GEMM1) and 4.5e-5 (GEMM2) of that sum, inside
#: 2^-14 = 6.1e-5.  Operands with a wide range inside a block do worse
#: (uniformly random codes: 1.9e-4; the worst case is 31 x 2^-13 of the block's
#: largest product), so the allowance is not a bound for arbitrary inputs.
MFMA_REL = 2.0 ** -14
F32_U = 2.0 ** -24  # unit roundoff of float32


def gemm_error_bound(a: np.ndarray, W: np.ndarray, rel: float = MFMA_REL) -> np.ndarray:
    """Bound on |h_gpu - h| for h = a W^T computed as one chain of K / 128
    block-scaled MFMA instructions per output, accumulating in float32.

    Model of one instruction D = C + (sum of its 128 products): the result is
    off by at most rel * (sum of the instruction's |products|) plus one
    float32 rounding of D.  Writing M for the sum of all |a_k W_k| of an
    output, every partial result is at most M (plus the errors so far), so
    after n instructions the error is at most
        rel M + n 2^-24 (M + rel M + error so far)  <=  (rel + n 2^-24 (1 + 4 rel)) M.
    ``a`` [rows, K] and ``W`` [outputs, K] are the dequantised operands.
    """
    K = a.shape[1]
    n = -(-K // 128)
    mag = np.abs(a) @ np.abs(W).T
    return (rel + n * F32_U * (1.0 + 4.0 * rel)) * mag


def swiglu_error_terms(h: np.ndarray, eh: np.ndarray, F: int) -> Dict[str, np.ndarray]:
    """Terms of a bound on |act_gpu - act| for act = silu(g) u, when the GPU's
    gate and up values are within eg, eu of g = h[:, :F], u = h[:, F:] and it
    evaluates act in float32.

    silu'' = s(1 - s)(2 + g(1 - 2s)) (s the sigmoid) never exceeds 1/2 in
    magnitude, so by the mean value theorem |silu(g + dg) - silu(g)| <=
    (|silu'(g)| + eg / 2) eg for |dg| <= eg, and
        |silu(g') u' - silu(g) u| <= |silu(g') - silu(g)| (|u| + eu) + |silu(g)| eu.
    Expanded:
      gate   |silu'(g)| |u| eg      first order in the gate error
      up     |silu(g)| eu           first order in the up error
      cross  |silu'(g)| eg eu       both errors at once
      curv   eg^2 / 2 (|u| + eu)    curvature of silu
      f32    float32 evaluation of silu(g) u from g and u: g log2(e), exp2,
             1 + e, reciprocal and two products, each within one or two
             float32 ulps, and the product's rounding shifts the exponent by
             |g| 2^-24, which scales e^-g by up to |g| 2^-24 relative:
             (10 + |g|) 2^-24 |act|; below g = -80 the float32 exponential
             overflows (or its reciprocal is subnormal) and silu may come out
             as 0: the whole |act|.
    """
    g, u = h[:, :F], h[:, F:]
    eg, eu = eh[:, :F], eh[:, F:]
    sg = sigmoid(g)
    dsilu = np.abs(sg * (1.0 + g * (1.0 - sg)))
    act = np.abs(g * sg * u)
    return dict(gate=dsilu * np.abs(u) * eg, up=np.abs(g * sg) * eu, cross=dsilu * eg * eu,
                curv=0.5 * eg * eg * (np.abs(u) + eu),
                f32=np.where(g < -80.0, act, (10.0 + np.abs(g)) * F32_U * act))


def act_error_bound(a: np.ndarray, w1: np.ndarray, w1s: np.ndarray, h: np.ndarray, F: int,
                    rel: float = MFMA_REL) -> np.ndarray:
    """A bound on |act_gpu - act| for the requant tie-zone test: the GEMM1
    accumulation bound (gemm_error_bound) carried through SwiGLU
    (swiglu_error_terms).  ``a`` are the dequantised input rows, ``h`` the
    oracle's float64 GEMM1 outputs."""
    eh = gemm_error_bound(a, fm.dequant_mxfp4(w1, w1s), rel)
    return sum(swiglu_error_terms(h, eh, F).values())
