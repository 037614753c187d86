"""Helpers of the GPU parity tests: upload a synth workload, run the HIP path
through the C ABI, and compare every stage with the CPU oracle.

Tolerances (the HIP path accumulates in f32, the oracle in f64):
  * integer stages (ids, phys, histogram, counts, offsets, row maps) and the
    activation quantisation (xq, xs): bit-exact;
  * routing weights: |w_gpu - w| <= 4e-6 |w| (sigmoid, sum and division in
    f32: a few ulps of 2^-24 each);
  * requantised act (aq, as): the GPU's code must be the RNE code of some
    value within the accumulation-error bound of the f64 act (the block-scaled
    MFMA rounds inside the instruction; measured worst case 2.5e-5 of the sum
    of absolute products, bound taken 2^-14), and its block exponent right
    for some amax within that bound; elsewhere this forces equality;
  * output: normwise relative error <= 1e-2 and elementwise relative error
    <= 5e-2 where |ref| > 1e-3, against the oracle's GEMM2 + combine applied
    to the GPU's own aq/as ("conditioned"), and normwise <= 1e-2 against the
    oracle's own end-to-end result.
"""

from __future__ import annotations

import numpy as np
import torch

import moe_expert_layer_sigmoid_amd as mx
from oracle import formats as fm
from oracle import moe as om

W_RTOL = 4e-6
OUT_NORM_TOL = 1e-2
OUT_ELEM_TOL = 5e-2
OUT_ELEM_FLOOR = 1e-3


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def upload(wl) -> dict:
    """Device copies of a workload; expert weights are packed by the library
    (moe_pack_weights) into w1..w2s, the natural MXFP4 bytes are not kept."""
    d = mx.Dims.of(wl.dims)
    nat = [dev(a) for a in (wl.w1, wl.w1s, wl.w2, wl.w2s)]
    packed = mx.pack_weights(d, *nat)
    del nat
    return dict(x=dev(wl.x.view(np.int16)), logits=dev(wl.logits), w1=packed[0], w1s=packed[1],
                w2=packed[2], w2s=packed[3], rep_count=dev(wl.rep_count.astype(np.int32)),
                rep_slots=dev(wl.rep_slots.astype(np.int32)))


def run_forward(wl, path="auto", buf=None, hist_init=None, taps=True, dims_kw=None):
    d = mx.Dims.of(wl.dims, **(dims_kw or {}))
    buf = buf or upload(wl)
    out = torch.full((max(d.T, 1), d.H), -1, dtype=torch.int16, device="cuda")
    hist = torch.zeros(d.P_total, dtype=torch.int32, device="cuda") if hist_init is None else hist_init
    ws = mx.workspace(d)
    tp = mx.make_taps(d) if taps else None
    chosen = mx.moe_forward(d, buf["x"], buf["logits"], buf["w1"], buf["w1s"], buf["w2"], buf["w2s"],
                            buf["rep_count"], buf["rep_slots"], out, ws, load_hist=hist, path=path, taps=tp)
    torch.cuda.synchronize()
    res = dict(out=out.cpu().numpy().view(np.uint16)[:d.T], hist=hist.cpu().numpy(), chosen=chosen)
    if tp is not None:
        TK = d.T * d.k
        c = {n: v.cpu().numpy() for n, v in tp.items()}
        rows = int(c["offsets"][d.P_local])
        res.update(topk_ids=c["topk_ids"][:TK].reshape(d.T, d.k), topk_w=c["topk_w"][:TK].reshape(d.T, d.k),
                   phys_ids=c["phys_ids"][:TK].reshape(d.T, d.k), counts=c["counts"][:d.P_local],
                   offsets=c["offsets"][:d.P_local + 1], rows=rows)
        nbh, nbf = d.H // 128, d.F // 128
        if chosen == "small_m":
            # pair-indexed intermediates; their bucket view follows from the GPU's
            # own phys: slot s's rows are its pairs in ascending (t, j) order
            phys = res["phys_ids"].ravel()
            por = np.concatenate([np.nonzero(phys == d.p0 + s)[0] for s in range(d.P_local)] +
                                 [np.zeros(0, np.int64)]).astype(np.int32)
            rop = np.full(TK, -1, np.int32)
            rop[por] = np.arange(len(por), dtype=np.int32)
            xq_tok = c["xq_tok"][:d.T * d.H].reshape(d.T, d.H)
            xs_tok = c["xs_tok"][:d.T * nbh].reshape(d.T, nbh)
            aq_pair = c["aq_pair"][:TK * d.F].reshape(TK, d.F)
            as_pair = c["as_pair"][:TK * nbf].reshape(TK, nbf)
            res.update(row_of_pair=rop, pair_of_row=por, xq_tok=xq_tok, xs_tok=xs_tok,
                       xq=xq_tok[por // d.k], xs=xs_tok[por // d.k], aq=aq_pair[por], as_=as_pair[por])
        else:
            res.update(row_of_pair=c["row_of_pair"][:TK], pair_of_row=c["pair_of_row"][:rows],
                       xq=c["xq"][:rows * d.H].reshape(rows, d.H),
                       xs=c["xs"][:rows * nbh].reshape(rows, nbh),
                       aq=c["aq"][:rows * d.F].reshape(rows, d.F),
                       as_=c["as_"][:rows * nbf].reshape(rows, nbf))
    return res


def oracle_front(wl) -> dict:
    """O1-O4 of the oracle (cheap at every size)."""
    d = wl.dims
    ids, w = om.route(wl.logits, d.k)
    phys, hist = om.remap_record(ids, wl.rep_count, wl.rep_slots, d.token_id_base, d.P_total)
    counts, offsets, rop, por = om.buckets(phys, d.p0, d.P_local)
    xq_t, xs_t = om.quant_blocks(fm.bf16_to_f64(wl.x))
    tok = por // d.k
    return dict(topk_ids=ids, topk_w=w, phys_ids=phys, load_hist=hist, counts=counts, offsets=offsets,
                row_of_pair=rop, pair_of_row=por, xq=xq_t[tok], xs=xs_t[tok], xq_tok=xq_t, xs_tok=xs_t)


def check_front(res, ref, d):
    assert np.array_equal(res["topk_ids"], ref["topk_ids"]), "topk_ids"
    assert np.all(np.abs(res["topk_w"] - ref["topk_w"]) <= W_RTOL * np.abs(ref["topk_w"])), "topk_w"
    assert np.array_equal(res["phys_ids"], ref["phys_ids"]), "phys_ids"
    assert np.array_equal(res["hist"], ref["load_hist"]), "load_hist"
    assert np.array_equal(res["counts"], ref["counts"]), "counts"
    assert np.array_equal(res["offsets"], ref["offsets"]), "offsets"
    assert np.array_equal(res["row_of_pair"], ref["row_of_pair"]), "row_of_pair"
    assert np.array_equal(res["pair_of_row"], ref["pair_of_row"]), "pair_of_row"
    assert np.array_equal(res["xs"], ref["xs"]), "xs"
    assert np.array_equal(res["xq"], ref["xq"]), "xq"
    if "xq_tok" in res:  # small-M: every token is quantised, local pairs or not
        assert np.array_equal(res["xs_tok"], ref["xs_tok"]), "xs_tok"
        assert np.array_equal(res["xq_tok"], ref["xq_tok"]), "xq_tok"


def _ordinal(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_aq_rows(aq_gpu, as_gpu, act, eps):
    """aq/as of some rows against the oracle's f64 act.

    The GPU's act differs from the f64 one by at most ``eps`` (elementwise), so
    a correct GPU picks, per 128-column block, an exponent that is right for
    some amax within max(eps) of the oracle's, and per element the RNE code of
    some value within eps of the oracle's (scaled by its own exponent).
    Returns (n_code_diffs, n_scale_diffs) for the report.
    """
    N, F = act.shape
    nb = F // 128
    blk = act.reshape(N, nb, 128)
    amax = np.abs(blk).max(-1)
    m = eps.reshape(N, nb, 128).max(-1)
    e_or = om.scale_exponent(amax)
    e_gpu = as_gpu.astype(np.int64) - 127
    e_lo = om.scale_exponent(np.maximum(amax - m, 0.0))
    e_hi = om.scale_exponent(amax + m)
    bad_s = (e_gpu < e_lo) | (e_gpu > e_hi)
    assert not bad_s.any(), f"scale outside its tie zone at {np.argwhere(bad_s)[:5].tolist()}"
    sc = np.ldexp(blk, (-e_gpu)[..., None]).reshape(N, F)
    tol = np.ldexp(eps.reshape(N, nb, 128), (-e_gpu)[..., None]).reshape(N, F)
    want = fm.enc_e4m3fn_rne(np.clip(sc, -448.0, 448.0))
    lo = _ordinal(fm.enc_e4m3fn_rne(np.clip(sc - tol, -448.0, 448.0)))
    hi = _ordinal(fm.enc_e4m3fn_rne(np.clip(sc + tol, -448.0, 448.0)))
    g = _ordinal(aq_gpu)
    ok = (g >= lo) & (g <= hi)
    if not np.all(ok):
        msg = []
        for r, c in np.argwhere(~ok)[:5]:
            e = int(e_gpu[r, c // 128])
            msg.append(f"row {r} col {c}: act {act[r, c]!r} e {e} scaled {sc[r, c]!r} "
                       f"oracle {fm.dec_e4m3fn(np.array([want[r, c]]))[0]} gpu {fm.dec_e4m3fn(np.array([aq_gpu[r, c]]))[0]} "
                       f"tol {tol[r, c]!r}")
        raise AssertionError("aq outside the tie zone:\n" + "\n".join(msg))
    return int((g != _ordinal(want)).sum()), int((e_gpu != e_or).sum())


def rel_errors(got: np.ndarray, ref: np.ndarray):
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    norm = num / den if den > 0 else num
    m = np.abs(ref) > OUT_ELEM_FLOOR
    elem = float(np.max(np.abs(got[m] - ref[m]) / np.abs(ref[m]))) if m.any() else 0.0
    return float(norm), elem


def check_out(out_gpu_bits, ref_f64, what="", bound=None):
    """Normwise and elementwise output checks.  With ``bound`` (an absolute
    error bound per element), an element also passes within that bound: for
    shapes whose outputs near the floor sit below the block-scaled MFMA's
    accumulation error (see y_error_bound)."""
    got = fm.bf16_to_f64(out_gpu_bits)
    norm, elem = rel_errors(got, ref_f64)
    assert norm <= OUT_NORM_TOL, f"{what} normwise {norm}"
    if bound is None:
        assert elem <= OUT_ELEM_TOL, f"{what} elementwise {elem}"
        return norm, elem
    err = np.abs(got - ref_f64)
    m = np.abs(ref_f64) > OUT_ELEM_FLOOR
    bad = m & (err > OUT_ELEM_TOL * np.abs(ref_f64)) & (err > bound)
    assert not bad.any(), (f"{what} elementwise {elem}, {int(bad.sum())} element(s) beyond both "
                           f"{OUT_ELEM_TOL} relative and the accumulation bound")
    return norm, elem


def y_error_bound(act_dq, w2, w2s):
    """A bound on |y_gpu - y| for GEMM2 rows on the same act: the oracle's
    bound for a chain of block-scaled MFMA instructions accumulating in
    float32 (oracle.moe.gemm_error_bound, the bound the GEMM1 tie-zone check
    carries through SwiGLU)."""
    return om.gemm_error_bound(act_dq, fm.dequant_mxfp4(w2, w2s))


def conditioned_bound(tokens, ref, yb, d, out_ref):
    """Error bound of the conditioned output: the combine of the y bounds with
    the routing weights, plus half a bf16 ulp (2^-8 relative) and a few f32
    ulps of the fma chain."""
    b = np.zeros((len(tokens), d.H))
    rop = ref["row_of_pair"].reshape(d.T, d.k)
    for i, t in enumerate(tokens):
        for j in range(d.k):
            r = int(rop[t, j])
            if r >= 0:
                b[i] += abs(ref["topk_w"][t, j]) * yb[r]
    return b + (2.0 ** -8 + 2.0 ** -20) * np.abs(out_ref)


def expert_check(wl, res, ref, slots, y_bounds=None):
    """GEMM1/requant of every row of ``slots`` against the oracle; returns the
    conditioned y rows (oracle GEMM2 on the GPU's aq/as) keyed by row (and
    fills ``y_bounds``, if given, with each row's y_error_bound)."""
    d = wl.dims
    y_c = {}
    stats = [0, 0]
    for s in slots:
        lo, hi = int(ref["offsets"][s]), int(ref["offsets"][s + 1])
        if hi == lo:
            continue
        a = om.dequant_blocks(ref["xq"][lo:hi], ref["xs"][lo:hi])
        act, h = om.gemm1_swiglu(a, wl.w1[s], wl.w1s[s], d.F)
        eps = om.act_error_bound(a, wl.w1[s], wl.w1s[s], h, d.F)
        nd, ns = check_aq_rows(res["aq"][lo:hi], res["as_"][lo:hi], act, eps)
        stats[0] += nd
        stats[1] += ns
        adq = om.dequant_blocks(res["aq"][lo:hi], res["as_"][lo:hi])
        y = om.gemm2(adq, wl.w2[s], wl.w2s[s])
        yb = y_error_bound(adq, wl.w2[s], wl.w2s[s]) if y_bounds is not None else None
        for i in range(hi - lo):
            y_c[lo + i] = y[i]
            if yb is not None:
                y_bounds[lo + i] = yb[i]
    return y_c, stats


def conditioned_out(tokens, ref, y_c, d):
    out = np.zeros((len(tokens), d.H))
    rop = ref["row_of_pair"].reshape(d.T, d.k)
    for i, t in enumerate(tokens):
        for j in range(d.k):
            r = int(rop[t, j])
            if r >= 0:
                out[i] += ref["topk_w"][t, j] * y_c[r]
    return out
