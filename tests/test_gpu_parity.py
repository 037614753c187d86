"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases are compared stage by stage in full; the full-size workloads
(T = 512 / 8192 with the 7168 x 2048 experts) are compared in full on every
integer stage and on the activation quantisation, and on sampled experts and
tokens for the GEMM stages (the oracle computes those one expert at a time).
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


def _full_check(wl, path="auto", acc_bound=False):
    """Every stage in full against the oracle's whole forward.  ``acc_bound``:
    an output element also passes within the GEMM2 accumulation bound."""
    d = wl.dims
    _say(f"[case] {wl.name} T={d.T} H={d.H} F={d.F} E={d.E} k={d.k} P={d.P_total}/{d.p0}+{d.P_local} path={path}")
    res = P.run_forward(wl, path=path)
    ref = P.oracle_front(wl)
    P.check_front(res, ref, d)
    yb = {} if acc_bound else None
    y_c, (nd, ns) = P.expert_check(wl, res, ref, range(d.P_local), yb)
    full = om.forward(wl)
    toks = list(range(d.T))
    cond = P.conditioned_out(toks, ref, y_c, d)
    bnd = P.conditioned_bound(toks, ref, yb, d, cond) if acc_bound else None
    n1 = P.check_out(res["out"], cond, "conditioned", bound=bnd)
    n2, _ = P.rel_errors(fm.bf16_to_f64(res["out"]), full["out"])
    assert n2 <= P.OUT_NORM_TOL, f"unconditioned normwise {n2}"
    # tokens without local pairs are exactly +0
    none_local = (ref["row_of_pair"].reshape(d.T, d.k) < 0).all(1)
    assert np.all(res["out"][none_local] == 0)
    _say(f"   ok: aq code diffs {nd}, scale diffs {ns}, out cond {n1}, uncond {n2:.2e}")
    return res


@pytest.mark.parametrize("path", ["auto", "small_m", "staged", "large_m"])
def test_tiny_all_paths(path):
    res = _full_check(synth.make("tiny"), path)
    assert res["chosen"] == ("small_m" if path == "auto" else path)


# With ~50 rows per slot, the large-input path runs its persistent tiled
# GEMMs (partial token blocks, and with F = H = 384 partial weight blocks).
@pytest.mark.parametrize("path", ["auto", "large_m"])
def test_mid_remote_pairs_and_ragged_tiles(path):
    # 200 tokens (ragged against 64-token chunks and 16-token tiles), half the
    # slots remote, ~50 rows per slot (several token tiles)
    _full_check(synth.make_custom(T=200, H=512, F=256, E=16, k=4, P_local=8, p0=4, seed=11), path)


@pytest.mark.parametrize("path", ["auto", "large_m"])
def test_odd_widths_and_eplb_replicas(path):
    # H/128 = 3 and F/128 = 3 (one 32-block group per lane, partial 256-row block
    # of H), replicas over 2 ranks, a non-zero global token id base
    _full_check(synth.make_custom(T=300, H=384, F=384, E=12, k=3, P_local=8, p0=8, redundant=4, ranks=2,
                                  seed=12, token_id_base=123456), path)


def test_tiled_several_token_blocks_per_slot():
    # ~250 rows per slot: two or three 128-token blocks per slot, the last
    # one ragged
    res = _full_check(synth.make_custom(T=1000, H=512, F=1024, E=16, k=4, P_local=8, p0=4, seed=22), "large_m")
    assert res["chosen"] == "large_m"


def test_tiled_skewed_slots():
    # Zipf popularity: the popular slots span up to five token blocks, the
    # rest one partial block
    wl = synth.make_custom(T=600, H=1024, F=512, E=16, k=4, P_local=8, p0=0, seed=23, zipf_s=1.2)
    res = _full_check(wl, "large_m")
    assert res["counts"].max() > 512 and res["chosen"] == "large_m"


@pytest.mark.parametrize("path", ["staged", "large_m"])
def test_bucket_ranks_when_every_pair_collides(path):
    # k = E = 16 over 24 slots (8 replicas): every token routes to every
    # expert, so a 64-token chunk holds 1024 pairs (sixteen 64-pair groups of
    # the bucketed count kernel) and each unreplicated slot gets 64 of them:
    # ranks 0..63 within every chunk, carried from group to group
    wl = synth.make_custom(T=200, H=256, F=256, E=16, k=16, P_local=10, p0=7, redundant=8, ranks=2, seed=31)
    res = _full_check(wl, path)
    assert res["counts"].max() == 200


# At the widest rows the outputs cover ~10^6 elements, and a few of those just
# above the elementwise floor (1e-3) sit below the block-scaled MFMA's own
# accumulation error; those elements are held to that bound (2^-14 of the
# sum of absolute products, the ratio the GEMM1 tie-zone check uses) instead
# of 5e-2 relative.  Weights are 0.02 scaled by sqrt(7168 / H) (W1) and
# sqrt(2048 / F) (W2), so pre-activations and outputs keep the decode share's
# magnitudes.
def _width_preserving(H, F):
    return (0.02 * (7168 / H) ** 0.5, 0.02 * (2048 / F) ** 0.5)


@pytest.mark.parametrize("H,F,path", [(16384, 256, "auto"), (16384, 256, "staged"),
                                      (256, 16384, "auto"), (256, 16384, "staged")])
def test_widest_rows_streaming(H, F, path):
    # the largest d_model / d_ff the library takes: 64 K steps of 256 in GEMM1
    # or GEMM2 through the streaming kernels
    _full_check(synth.make_custom(T=64, H=H, F=F, E=8, k=2, P_local=8, seed=24 if H > F else 25,
                                  w_std=_width_preserving(H, F)), path, acc_bound=True)


@pytest.mark.parametrize("H,F", [(8192, 512), (512, 8192)])
def test_widest_rows_tiled(H, F):
    # ~64 rows per slot at the tiled kernels' K limit (64 stages of 128)
    res = _full_check(synth.make_custom(T=256, H=H, F=F, E=8, k=2, P_local=8, seed=26 if H > F else 27,
                                        w_std=_width_preserving(H, F)), "large_m", acc_bound=True)
    assert res["chosen"] == "large_m"


@pytest.mark.parametrize("E,k,T", [(384, 6, 203), (1024, 16, 37), (40, 3, 17)])
def test_routing_identical_on_both_fronts(E, k, T):
    # the fused small-input front routes one token per wavefront, the routing
    # pass of the bucketed paths one token per 16-lane row: the same choices
    # and the same weights, bit for bit (ragged last rows included)
    wl = synth.make_custom(T=T, H=256, F=128, E=E, k=k, P_local=8, p0=0, seed=41)
    a = P.run_forward(wl, path="small_m")
    b = P.run_forward(wl, path="large_m")
    assert a["chosen"] == "small_m" and b["chosen"] == "large_m"
    for n in ("topk_ids", "topk_w", "phys_ids"):
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("path", ["auto", "staged"])
def test_wide_k_and_many_experts(path):
    # k = 16 of 1024 experts (16 logits per lane), skewed popularity; staged:
    # the bucketed count kernel's LDS histogram at its largest table (1024)
    _full_check(synth.make_custom(T=96, H=256, F=128, E=1024, k=16, P_local=64, p0=0, seed=13, zipf_s=1.2), path)


def test_single_token_and_capacity_bucket():
    wl = synth.make_custom(T=1, H=256, F=128, E=8, k=2, P_local=8, seed=14, T_max=512)
    _full_check(wl)


@pytest.mark.parametrize("path", ["auto", "staged"])
def test_few_touched_slots(path):
    # fewer pairs than slots: most GEMM blocks find their slot empty and
    # return at once (H = 3072: 12 GEMM2 blocks of 256 rows per slot)
    _full_check(synth.make_custom(T=8, H=3072, F=512, E=64, k=6, P_local=16, p0=8, seed=21), path)


def test_decode_split_k_many_touched_slots():
    # 8 tokens whose 16 experts all lie among this GPU's 32 local slots (of
    # 512): the decode-share form splits K in both GEMMs and runs 16 block
    # rows for the ~32 touched slots, so that a row takes several slots in turn
    wl = synth.make_custom(T=8, H=2048, F=2048, E=512, k=16, P_local=32, p0=0, seed=31)
    wl.logits[:, 32:] = -30.0
    res = _full_check(wl, "small_m")
    assert len(np.unique(res["phys_ids"])) > 16
    again = P.run_forward(wl, path="small_m")
    assert np.array_equal(res["out"], again["out"])


def test_small_m_at_its_token_limit():
    # 1024 tokens each routed to all 16 experts: every slot lists 1024 pairs,
    # the small-input path's capacity
    wl = synth.make_custom(T=1024, H=256, F=128, E=16, k=16, P_local=16, seed=20)
    res = _full_check(wl, "small_m")
    assert res["rows"] == 1024 * 16


def test_all_pairs_remote_gives_zero_output():
    wl = synth.make_custom(T=40, H=256, F=128, E=16, k=2, P_local=4, p0=12, seed=15)
    wl.logits[:, 12:] = -30.0          # nobody picks experts 12..15
    res = _full_check(wl)
    assert res["rows"] == 0 and np.all(res["out"] == 0)


def test_zero_tokens_writes_nothing():
    wl = synth.make_custom(T=0, H=256, F=128, E=8, k=2, P_local=8, seed=16, T_max=64)
    d = mx.Dims.of(wl.dims)
    buf = P.upload(synth.make_custom(T=1, H=256, F=128, E=8, k=2, P_local=8, seed=16))
    out = torch.full((4, d.H), 7, dtype=torch.int16, device="cuda")
    hist = torch.zeros(d.P_total, dtype=torch.int32, device="cuda")
    mx.moe_forward(d, buf["x"], buf["logits"], buf["w1"], buf["w1s"], buf["w2"], buf["w2s"], buf["rep_count"],
                   buf["rep_slots"], out, mx.workspace(d), load_hist=hist)
    torch.cuda.synchronize()
    assert torch.all(out == 7) and torch.all(hist == 0)


@pytest.mark.parametrize("path", ["small_m", "staged"])
def test_component_calls_match_forward_bitwise(path):
    # the pair-indexed small-input path and the bucketed component calls run
    # the same arithmetic in the same order: equal bit for bit
    wl = synth.make_custom(T=130, H=512, F=256, E=16, k=4, P_local=8, p0=4, redundant=8, ranks=2, seed=17)
    d = mx.Dims.of(wl.dims)
    buf = P.upload(wl)
    res = P.run_forward(wl, buf=buf, path=path)
    TK, TMK = d.T * d.k, d.T_max * d.k
    z = lambda n, dt: torch.zeros(n, dtype=dt, device="cuda")  # noqa: E731
    ids, w, phys = z(TK, torch.int32), z(TK, torch.float32), z(TK, torch.int32)
    hist = z(d.P_total, torch.int32)
    counts, offsets = z(d.P_local, torch.int32), z(d.P_local + 1, torch.int32)
    rop, por = z(TK, torch.int32), z(TMK, torch.int32)
    xq, xs = z(TMK * d.H, torch.uint8), z(TMK * d.H // 128, torch.uint8)
    aq, as_ = z(TMK * d.F, torch.uint8), z(TMK * d.F // 128, torch.uint8)
    out = torch.full((d.T, d.H), -1, dtype=torch.int16, device="cuda")
    ws = mx.workspace(d)
    mx.moe_route(d, buf["logits"], ids, w)
    mx.moe_eplb_remap_record(d, ids, buf["rep_count"], buf["rep_slots"], phys, hist, ws)
    mx.moe_quant_permute(d, buf["x"], phys, xq, xs, counts, offsets, rop, por, ws)
    mx.moe_grouped_gemm1_swiglu(d, xq, xs, offsets, buf["w1"], buf["w1s"], aq, as_, ws)
    mx.moe_grouped_gemm2_combine(d, aq, as_, offsets, buf["w2"], buf["w2s"], rop, w, out, ws)
    torch.cuda.synchronize()
    rows = res["rows"]
    assert np.array_equal(ids.cpu().numpy().reshape(d.T, d.k), res["topk_ids"])
    assert np.array_equal(w.cpu().numpy().reshape(d.T, d.k), res["topk_w"])
    assert np.array_equal(phys.cpu().numpy().reshape(d.T, d.k), res["phys_ids"])
    assert np.array_equal(hist.cpu().numpy(), res["hist"])
    assert np.array_equal(offsets.cpu().numpy(), res["offsets"])
    assert np.array_equal(por.cpu().numpy()[:rows], res["pair_of_row"])
    assert np.array_equal(aq.cpu().numpy()[:rows * d.F].reshape(rows, d.F), res["aq"])
    assert np.array_equal(out.cpu().numpy().view(np.uint16), res["out"])


def test_pair_components_match_small_m_forward_bitwise():
    wl = synth.make_custom(T=130, H=512, F=256, E=16, k=4, P_local=8, p0=4, redundant=8, ranks=2, seed=17)
    d = mx.Dims.of(wl.dims)
    buf = P.upload(wl)
    tp = mx.make_taps(d)
    out_f = torch.full((d.T, d.H), -1, dtype=torch.int16, device="cuda")
    mx.moe_forward(d, buf["x"], buf["logits"], buf["w1"], buf["w1s"], buf["w2"], buf["w2s"], buf["rep_count"],
                   buf["rep_slots"], out_f, mx.workspace(d), path="small_m", taps=tp)
    TK = d.T * d.k
    z = lambda n, dt: torch.zeros(n, dtype=dt, device="cuda")  # noqa: E731
    aq, as_ = z(TK * d.F, torch.uint8), z(TK * d.F // 128, torch.uint8)
    counts, offsets = z(d.P_local, torch.int32), z(d.P_local + 1, torch.int32)
    out = torch.full((d.T, d.H), -1, dtype=torch.int16, device="cuda")
    mx.moe_grouped_gemm1_swiglu_pairs(d, tp["xq_tok"], tp["xs_tok"], tp["phys_ids"], buf["w1"], buf["w1s"], aq, as_,
                                      counts)
    mx.moe_grouped_gemm2_combine_pairs(d, aq, as_, tp["phys_ids"], buf["w2"], buf["w2s"], tp["topk_w"], counts,
                                       offsets, out, mx.workspace(d))
    torch.cuda.synchronize()
    local = np.isin(tp["phys_ids"].cpu().numpy()[:TK], np.arange(d.p0, d.p0 + d.P_local))
    assert np.array_equal(counts.cpu().numpy(), tp["counts"].cpu().numpy())
    assert np.array_equal(offsets.cpu().numpy(), tp["offsets"].cpu().numpy())
    a1 = aq.cpu().numpy().reshape(TK, d.F)[local]
    a2 = tp["aq_pair"].cpu().numpy()[:TK * d.F].reshape(TK, d.F)[local]
    assert np.array_equal(a1, a2)
    assert np.array_equal(out.cpu().numpy(), out_f.cpu().numpy())


def test_deterministic_and_histogram_accumulates():
    wl = synth.make_custom(T=257, H=256, F=128, E=32, k=6, P_local=16, p0=8, redundant=8, ranks=2, seed=18)
    d = mx.Dims.of(wl.dims)
    buf = P.upload(wl)
    hist = torch.zeros(d.P_total, dtype=torch.int32, device="cuda")
    a = P.run_forward(wl, buf=buf, hist_init=hist)
    b = P.run_forward(wl, buf=buf, hist_init=hist)
    for n in ("out", "topk_w", "aq", "as_", "xq", "pair_of_row"):
        assert np.array_equal(a[n], b[n]), n
    ref = P.oracle_front(wl)
    assert np.array_equal(hist.cpu().numpy(), 2 * ref["load_hist"])
    assert hist.cpu().numpy().sum() == 2 * d.T * d.k


def test_quant_every_bf16_value():
    """Every finite bf16 pattern goes through the activation quantiser."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    H = 1024
    T = (bits.size + H - 1) // H
    x = np.zeros(T * H, np.uint16)
    x[:bits.size] = bits
    rng = np.random.default_rng(0)
    x = x[rng.permutation(x.size)].reshape(T, H)   # mix magnitudes inside blocks
    wl = synth.make_custom(T=T, H=H, F=128, E=4, k=1, P_local=4, seed=19)
    wl.x = x
    d = mx.Dims.of(wl.dims)
    buf = P.upload(wl)
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")    # every token to expert 0
    rop, por = torch.zeros(T, dtype=torch.int32, device="cuda"), torch.zeros(T, dtype=torch.int32, device="cuda")
    xq = torch.zeros(T * H, dtype=torch.uint8, device="cuda")
    xs = torch.zeros(T * H // 128, dtype=torch.uint8, device="cuda")
    counts = torch.zeros(4, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(5, dtype=torch.int32, device="cuda")
    mx.moe_quant_permute(d, buf["x"], ids, xq, xs, counts, offsets, rop, por, mx.workspace(d))
    torch.cuda.synchronize()
    q, s = om.quant_blocks(fm.bf16_to_f64(x))
    assert np.array_equal(xs.cpu().numpy().reshape(T, -1), s)
    assert np.array_equal(xq.cpu().numpy().reshape(T, H), q)


# ---------------------------------------------------------------------------- full size

def _big_check(wl, n_slots=3, n_tokens=24, path="auto", buf=None):
    d = wl.dims
    _say(f"[case] {wl.name} T={d.T} path={path}")
    res = P.run_forward(wl, path=path, buf=buf)
    ref = P.oracle_front(wl)
    P.check_front(res, ref, d)
    rng = np.random.default_rng(d.T)
    toks = np.sort(rng.choice(d.T, size=min(n_tokens, d.T), replace=False))
    rop = ref["row_of_pair"].reshape(d.T, d.k)
    slots = set(rng.choice(d.P_local, size=n_slots, replace=False).tolist())
    for t in toks:
        for j in range(d.k):
            if rop[t, j] >= 0:
                slots.add(int(ref["phys_ids"][t, j]) - d.p0)
    y_c, (nd, ns) = P.expert_check(wl, res, ref, sorted(slots))
    cond = P.conditioned_out(toks, ref, y_c, d)
    n1 = P.check_out(res["out"][toks], cond, "conditioned")
    unc = np.stack([om.forward_token(wl, int(t)) for t in toks[:8]])
    n2, _ = P.rel_errors(fm.bf16_to_f64(res["out"][toks[:8]]), unc)
    assert n2 <= P.OUT_NORM_TOL
    _say(f"   ok: {len(slots)} slots, aq code diffs {nd}, scale diffs {ns}, out cond {n1}, uncond {n2:.2e}")
    return res


@pytest.mark.parametrize("path", ["auto", "staged"])
def test_decode_share_512_tokens(path):
    res = _big_check(synth.make("decode512"), path=path)
    assert res["chosen"] == ("small_m" if path == "auto" else path)


def test_prefill_share_8192_tokens():
    res = _big_check(synth.make("prefill8192"))
    assert res["chosen"] == "large_m"


def test_sweep_16384_tokens():
    # 256 mean rows per slot: two or three token blocks per slot at full width
    res = _big_check(synth.make_sweep(16384), n_slots=2, n_tokens=8)
    assert res["chosen"] == "large_m"


@pytest.mark.parametrize("T", [1, 8, 1024, 4096])
def test_sweep_points_at_full_width(T):
    """Sweep points at d_model 7168 / d_ff 2048: one and eight tokens (the
    small-input path with few touched experts), 1024 tokens (the large-input
    path still streaming weights: 16 rows per slot, two 16-row token tiles per
    pass) and 4096 (the tiled kernels with half-filled 128-token blocks and a
    partial last round of items)."""
    res = _big_check(synth.make_sweep(T), n_slots=2, n_tokens=12)
    assert res["chosen"] == ("small_m" if T <= 512 else "large_m")


def test_prefill_ep8_rank_share_65536_tokens():
    """The EP-shaped prefill share the benchmark times (8 ranks x 8192 tokens
    routed into this GPU's 48 experts, ~1030 rows per slot: nine 128-token
    blocks per slot on the tiled kernels), compared like the other full-size
    workloads."""
    wl = synth.make_ep_shaped(8)
    res = _big_check(wl, n_slots=2, n_tokens=12, path="large_m")
    assert res["chosen"] == "large_m" and res["rows"] > 45000


def test_skewed_routing_with_eplb_8192_tokens():
    wl = synth.make("eplb8192")
    res = _big_check(wl)
    # the recorder saw every pair, on all 448 physical slots
    assert res["hist"].sum() == wl.dims.T * wl.dims.k and wl.dims.P_total == 448


@pytest.mark.parametrize("path", ["small_m", "staged"])
def test_padded_k_ignores_workspace_bytes(path):
    """d_model 512 and d_ff 256 pad K to 1024 in the packed weights: the
    padded steps must read zero tokens, whatever the workspace holds (here
    every byte 0x7F, an fp8 NaN code) -- a regression case."""
    wl = synth.make_custom(T=64, H=512, F=256, E=384, k=6, P_local=48, seed=410)
    d = mx.Dims.of(wl.dims)
    _say(f"[case] padded K, workspace of NaN codes, path={path}")
    buf = P.upload(wl)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device="cuda")
    ws = torch.full((mx.moe_workspace_bytes(d),), 0x7F, dtype=torch.uint8, device="cuda")
    mx.moe_forward(d, buf["x"], buf["logits"], buf["w1"], buf["w1s"], buf["w2"], buf["w2s"], buf["rep_count"],
                   buf["rep_slots"], out, ws, path=path)
    torch.cuda.synchronize()
    got = fm.bf16_to_f64(out.cpu().numpy().view(np.uint16))
    assert np.all(np.isfinite(got))
    n2, _ = P.rel_errors(got, om.forward(wl)["out"])
    assert n2 <= P.OUT_NORM_TOL, n2
    _say(f"   ok: normwise {n2:.2e}")
