#!/usr/bin/env python3
"""Benchmark: MoE-layer tokens/s of one MI355X's share of the fused MoE layer.

One step = one ``moe_forward`` (route, EPLB remap, quant + dispatch, GEMM1 +
SwiGLU + requant, GEMM2, combine) over one batch of seeded synthetic inputs.
The headline is the decode share: 512 tokens, d_model 7168, d_ff 2048, 384
experts, top-6 sigmoid routing, 48 local experts (one EP8 rank's share), fp8
activations on MXFP4 experts.  The same line carries the 8192-token half of
the metric: the literal prefill share (8192 tokens into the same 48 experts)
and the EP-shaped prefill share (8 ranks x 8192 tokens routed into this
GPU's 48 experts, the load an EP8 rank's experts see), each with the GEMM
kernels' times measured inside the timed forwards.  Inputs are resident in
HBM before each timed region; the expert weights rotate over several device
copies so that no step finds them in the 256 MB MALL or in L2.

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this build runs on one
GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA, published
ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = ("moe_expert_layer_sigmoid_amd/csrc/kernels_gemm.hip",
                "moe_expert_layer_sigmoid_amd/csrc/moe_device.hpp",
                "moe_expert_layer_sigmoid_amd/csrc/moe_layout.hpp",
                "moe_expert_layer_sigmoid_amd/csrc/moe_pairs.hpp")


def _src_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def w1_bytes(d, touched: int) -> int:
    """Algorithmic bytes of GEMM1's weights: MXFP4 W1 + scales of every
    touched slot (15,597,568 B per slot at d_model 7168, d_ff 2048)."""
    return touched * (2 * d.F * d.H // 2 + 2 * d.F * d.H // 32)


def w2_bytes(d, touched: int) -> int:
    """Algorithmic bytes of GEMM2's weights: MXFP4 W2 + scales of every touched slot."""
    return touched * (d.H * d.F // 2 + d.H * d.F // 32)


def layer_bytes(d, touched: int) -> int:
    """Algorithmic bytes of the layer: all weights of touched slots, and per token
    its logits (f32), input row and output row (bf16)."""
    return w1_bytes(d, touched) + w2_bytes(d, touched) + d.T * (d.E * 4 + d.H * 2 + d.H * 2)


def layer_flops(d, rows: int) -> int:
    """Algorithmic flop: 2 (2F H + H F) per local (token, expert) pair."""
    return 2 * rows * (2 * d.F * d.H + d.H * d.F)


def packed_weights(wl, copies: int):
    """The workload's experts packed once (outside every timed region), plus
    copies - 1 clones to rotate over."""
    import torch
    import moe_expert_layer_sigmoid_amd as mx
    d = mx.Dims.of(wl.dims)
    nat = [torch.from_numpy(a).to("cuda") for a in (wl.w1, wl.w1s, wl.w2, wl.w2s)]
    w = [mx.pack_weights(d, *nat)]
    del nat
    for _ in range(copies - 1):
        w.append(tuple(t.clone() for t in w[0]))
    return w


def measure(wl, weights, steps: int, warmup: int, path: str = "auto"):
    """Time `steps` forwards of workload ``wl`` after `warmup`, the weights
    rotating over ``weights``: first plain forwards (the step time), then
    `steps` more that also record HIP events right before and after their
    GEMM1 and GEMM2 launches (on the stream the kernels run on), which give
    the GEMM kernels' times inside whole forwards (the events are kept out
    of the first region: four records inside a forward cost about 10 us of
    step time).  Returns a dict of the measurements."""
    import torch
    import moe_expert_layer_sigmoid_amd as mx

    d = mx.Dims.of(wl.dims)
    dev = "cuda"
    x = torch.from_numpy(wl.x.view("int16")).to(dev)
    logits = torch.from_numpy(wl.logits).to(dev)
    rc = torch.from_numpy(wl.rep_count).to(dev)
    rs = torch.from_numpy(wl.rep_slots).to(dev)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=dev)
    ws = mx.workspace(d)
    taps = mx.make_taps(d)
    chosen = mx.moe_forward(d, x, logits, *weights[0], rc, rs, out, ws, taps=taps, path=path)
    torch.cuda.synchronize()
    counts = taps["counts"].cpu().numpy()
    touched, rows = int((counts > 0).sum()), int(counts.sum())
    del taps
    nw = len(weights)
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for e in [e for four in ev for e in four]:
        e.record(st)        # creates the HIP event behind each torch event
    for i in range(warmup):
        mx.moe_forward(d, x, logits, *weights[i % nw], rc, rs, out, ws, path=path)
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    for i in range(steps):
        marks[i].record(st)
        mx.moe_forward(d, x, logits, *weights[i % nw], rc, rs, out, ws, path=path)
    marks[steps].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw0
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    for i in range(steps):
        mx.moe_forward(d, x, logits, *weights[i % nw], rc, rs, out, ws, path=path, gemm_events=ev[i])
    torch.cuda.synchronize()
    g1 = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)) / steps
    g2 = sum(ev[i][2].elapsed_time(ev[i][3]) for i in range(steps)) / steps
    del ws, out
    torch.cuda.empty_cache()
    return dict(d=d, chosen=chosen, touched=touched, rows=rows, wall=wall,
                gpu_ms=marks[0].elapsed_time(marks[steps]), per_step=per_step,
                gemm1_us=g1 * 1000.0, gemm2_us=g2 * 1000.0)


def copy_rate_gbs() -> float:
    """Achievable HBM rate: a plain 1 GiB device-to-device copy (read + write)."""
    import torch
    st = torch.cuda.current_stream()
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(st)
    for _ in range(5):
        dst.copy_(src)
    c1.record(st)
    torch.cuda.synchronize()
    return 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9


def summary(r, label: str):
    """Per-workload figures: tokens/s, fractions of the HBM roofline (layer
    bytes) and of the MFMA peak (layer flop), the GEMM kernels' times."""
    d = r["d"]
    ms = r["gpu_ms"] / len(r["per_step"])
    lay, fl = layer_bytes(d, r["touched"]), layer_flops(d, r["rows"])
    g1, g2 = r["gemm1_us"] * 1e-6, r["gemm2_us"] * 1e-6
    f1 = 2 * r["rows"] * 2 * d.F * d.H
    return {"workload": label, "T": d.T, "path": r["chosen"], "touched_slots": r["touched"], "rows": r["rows"],
            "ms_per_step": round(ms, 4), "tokens_per_s": round(d.T / (ms * 1e-3), 1),
            "hbm_frac": round(lay / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
            "gemm1_us": round(r["gemm1_us"], 2), "gemm2_us": round(r["gemm2_us"], 2),
            "gemm1_mfma_frac": round(f1 / g1 / 1e12 / FP8_PEAK_TFLOPS, 4),
            "gemm2_mfma_frac": round((fl - f1) / g2 / 1e12 / FP8_PEAK_TFLOPS, 4),
            "gemms_mfma_frac": round(fl / (g1 + g2) / 1e12 / FP8_PEAK_TFLOPS, 4),
            "gemm1_weight_gbs": round(w1_bytes(d, r["touched"]) / g1 / 1e9, 1),
            "gemm2_weight_gbs": round(w2_bytes(d, r["touched"]) / g2 / 1e9, 1)}


def _time(fn, steps: int, warmup: int, stream) -> float:
    """Average milliseconds of fn(i) over `steps` calls after `warmup`, by
    events on the stream the work is launched on."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_sweep(steps: int, warmup: int, copies: int, only=None):
    """The token-count sweep (decode-share shapes, AUTO path at each T), the
    EP-shaped prefill share (8 ranks x 8192 tokens into this GPU's 48
    experts, LARGE_M) and the skewed-routing EPLB share (8192 tokens, 448
    physical slots, 56 local).  One JSON line per point on stdout."""
    import torch
    import synth

    w = packed_weights(synth.make_sweep(1), copies)

    def point(wl, name, path="auto", wts=None, extra=None):
        r = measure(wl, w if wts is None else wts, steps, warmup, path)
        rec = {"point": name, **summary(r, name)}
        rec.pop("workload")
        if extra:
            rec.update(extra(r["d"], rec["ms_per_step"]))
        print(json.dumps(rec), flush=True)

    for T in synth.SWEEP_T:
        if only is None or f"sweep_T{T}" in only:
            point(synth.make_sweep(T, with_weights=False), f"sweep_T{T}")
    if only is None or "prefill_ep8_rank_share" in only:
        # tokens/s of one rank's share: its 8192 tokens per whole call
        point(synth.make_ep_shaped(8, with_weights=False), "prefill_ep8_rank_share", path="large_m",
              extra=lambda d, ms: {"rank_share_tokens_per_s": round(8192 / (ms * 1e-3), 1)})
    if only is None or "eplb8192" in only:
        del w[1:]
        torch.cuda.empty_cache()
        wl = synth.make("eplb8192")
        we = packed_weights(wl, copies)
        point(wl, "eplb8192", wts=we, extra=lambda d, ms: {"P_total": d.P_total, "P_local": d.P_local})
        del we
        torch.cuda.empty_cache()
    if only is None or "eplb_migrate448" in only:
        eplb_migrate_point(steps, warmup)
    for T in (512, 8192):
        if only is None or f"router_T{T}" in only:
            router_point(T, steps, warmup)
    if only is None or "graph_T512" in only:
        graph_point(steps, warmup)
    if only is None or "a16w4_T512" in only:
        a16w4_point(steps, warmup)


def a16w4_point(steps: int, warmup: int):
    """The a16w4 variant (bf16 activations on the MXFP4 experts) at the decode
    share's shapes, weights rotated over 3 copies: tokens/s and the fraction of
    the layer's HBM roofline (the same algorithmic bytes as the a8w4 layer)."""
    import torch
    import moe_expert_layer_sigmoid_amd as mx
    import synth

    dev = "cuda"
    st = torch.cuda.current_stream()
    wl = synth.make("decode512")
    d = mx.Dims.of(wl.dims)
    nat = [torch.from_numpy(a).to(dev) for a in (wl.w1, wl.w1s, wl.w2, wl.w2s)]
    w = [mx.pack_weights(d, *nat)]
    del nat
    for _ in range(2):
        w.append(tuple(t.clone() for t in w[0]))
    x = torch.from_numpy(wl.x.view("int16")).to(dev)
    logits = torch.from_numpy(wl.logits).to(dev)
    rc = torch.from_numpy(wl.rep_count).to(dev)
    rs = torch.from_numpy(wl.rep_slots).to(dev)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=dev)
    ws = mx.a16w4_workspace(d)
    ms = _time(lambda i: mx.moe_forward_a16w4(d, x, logits, *w[i % 3], rc, rs, out, ws), steps, warmup, st)
    touched = 48
    lay = layer_bytes(d, touched)
    rec = {"point": "a16w4_T512", "T": d.T, "ms_per_step": round(ms, 4), "tokens_per_s": round(d.T / (ms * 1e-3), 1),
           "hbm_frac": round(lay / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    print(json.dumps(rec), flush=True)


def graph_point(steps: int, warmup: int):
    """The decode share (512 tokens) as one captured HIP graph of the
    device-count small-input call (moe_forward_small_m, bucket 512): replay
    time with all 512 tokens valid and for an idle step (0 valid), next to
    the eager moe_forward, weights rotated over 3 copies in both."""
    import torch
    import moe_expert_layer_sigmoid_amd as mx
    import synth

    dev = "cuda"
    st = torch.cuda.current_stream()
    wl = synth.make("decode512")
    d = mx.Dims.of(wl.dims)
    nat = [torch.from_numpy(a).to(dev) for a in (wl.w1, wl.w1s, wl.w2, wl.w2s)]
    w = [mx.pack_weights(d, *nat)]
    del nat
    for _ in range(2):
        w.append(tuple(t.clone() for t in w[0]))
    x = torch.from_numpy(wl.x.view("int16")).to(dev)
    logits = torch.from_numpy(wl.logits).to(dev)
    rc = torch.from_numpy(wl.rep_count).to(dev)
    rs = torch.from_numpy(wl.rep_slots).to(dev)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=dev)
    ws = mx.workspace(d)
    nt = torch.tensor([d.T], dtype=torch.int32, device=dev)
    eager = _time(lambda i: mx.moe_forward(d, x, logits, *w[i % 3], rc, rs, out, ws, path="small_m"), steps,
                  warmup, st)
    side = torch.cuda.Stream()
    side.wait_stream(st)
    with torch.cuda.stream(side):
        for i in range(3):
            mx.moe_forward_small_m(d, nt, x, logits, *w[i], rc, rs, out, ws)
    st.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(3):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            mx.moe_forward_small_m(d, nt, x, logits, *w[i], rc, rs, out, ws)
        graphs.append(g)
    torch.cuda.synchronize()
    full = _time(lambda i: graphs[i % 3].replay(), steps, warmup, st)
    nt.fill_(0)
    idle = _time(lambda i: graphs[i % 3].replay(), steps, warmup, st)
    rec = {"point": "graph_T512", "T": d.T, "eager_ms": round(eager, 4), "graph_ms": round(full, 4),
           "graph_idle_ms": round(idle, 4), "tokens_per_s_graph": round(d.T / (full * 1e-3), 1)}
    print(json.dumps(rec), flush=True)


BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, published


def router_point(T: int, steps: int, warmup: int):
    """Router projection (moe_router_logits) at the decode / prefill shares'
    router shape: x bf16 [T, 7168] times a bf16 gate [384, 7168] -> f32
    logits.  Algorithmic bytes: x, the gate and the logits once; flop 2 T E H."""
    import numpy as np
    import torch
    import moe_expert_layer_sigmoid_amd as mx
    import synth

    dev = "cuda"
    st = torch.cuda.current_stream()
    H, E = 7168, 384
    wl = synth.make_sweep(T, with_weights=False)
    d = mx.Dims.of(wl.dims)
    x = torch.from_numpy(wl.x.view("int16")).to(dev)
    wg = torch.from_numpy(synth.gate_weights(1, E, H).view(np.int16)).to(dev)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    ws = mx.router_workspace(d)
    ms = _time(lambda i: mx.moe_router_logits(d, x, wg, lg, ws, stream=st), steps, warmup, st)
    nbytes = T * H * 2 + E * H * 2 + T * E * 4
    flops = 2 * T * E * H
    t = ms * 1e-3
    hbm, mfma = nbytes / t / 1e9 / HBM_PEAK_GBS, flops / t / 1e12 / BF16_PEAK_TFLOPS
    rec = {"point": f"router_T{T}", "T": T, "H": H, "E": E, "ms": round(ms, 4),
           "tokens_per_s": round(T / t, 1), "hbm_frac": round(hbm, 4), "mfma_bf16_frac": round(mfma, 4),
           "roofline_frac": round(max(hbm, mfma), 4), "bound": "hbm" if hbm >= mfma else "mfma"}
    print(json.dumps(rec), flush=True)


def eplb_migrate_point(steps: int, warmup: int):
    """EPLB rebalance + weight migration on the skewed share's shape: record
    the loads of 8192 Zipf-routed tokens on the naive 448-slot table with the
    fused forward, rebalance (library host call, timed on the host), and time
    the migration kernel that copies the new experts of rank 0's 56 slots
    from a pool of all 384 packed experts (copy time does not depend on the
    bytes, so the pool is zero-filled)."""
    import numpy as np
    import torch
    import moe_expert_layer_sigmoid_amd as mx
    import synth

    dev = "cuda"
    st = torch.cuda.current_stream()
    c = synth.WORKLOADS["eplb8192"]
    wl = synth.make("eplb8192", with_weights=False)
    E, Pt, ranks = wl.dims.E, wl.dims.P_total, c["ranks"]
    rc0, rs0, se0 = synth.naive_replica_map(E, Pt)
    d = mx.Dims.of(wl.dims, R_max=rs0.shape[1])
    per = [mx.moe_packed_bytes(d, i) // d.P_local for i in range(4)]
    slots = [torch.zeros(per[i] * d.P_local, dtype=torch.uint8, device=dev) for i in range(4)]
    hist = torch.zeros(Pt, dtype=torch.int32, device=dev)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=dev)
    mx.moe_forward(d, torch.from_numpy(wl.x.view("int16")).to(dev), torch.from_numpy(wl.logits).to(dev),
                   *slots, torch.from_numpy(rc0).to(dev), torch.from_numpy(rs0).to(dev), out, mx.workspace(d),
                   load_hist=hist)
    h = hist.cpu().numpy()
    t0 = time.perf_counter()
    rc1, rs1, se1 = mx.moe_eplb_rebalance(E, Pt, ranks, 64, h, se0)
    host_ms = (time.perf_counter() - t0) * 1e3
    loc = slice(d.p0, d.p0 + d.P_local)
    src_np = np.where(se0[loc] == se1[loc], -1, se1[loc]).astype(np.int32)
    moved = int((src_np >= 0).sum())
    src = torch.from_numpy(src_np).to(dev)
    pool = [torch.zeros(per[i] * E, dtype=torch.uint8, device=dev) for i in range(4)]
    ms = _time(lambda i: mx.moe_eplb_migrate(d, src, E, pool, slots, stream=st), steps, warmup, st)
    nbytes = 2 * moved * sum(per)
    # the recorded batch's largest slot load before and after (same tokens)
    after = torch.zeros(Pt, dtype=torch.int32, device=dev)
    mx.moe_forward(mx.Dims.of(d, R_max=rs1.shape[1]), torch.from_numpy(wl.x.view("int16")).to(dev),
                   torch.from_numpy(wl.logits).to(dev), *slots, torch.from_numpy(rc1).to(dev),
                   torch.from_numpy(rs1).to(dev), out, mx.workspace(d), load_hist=after)
    rec = {"point": "eplb_migrate448", "T": d.T, "P_total": Pt, "P_local": d.P_local, "moved_slots": moved,
           "rebalance_host_ms": round(host_ms, 3), "migrate_ms": round(ms, 4),
           "migrate_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "max_slot_load_before": int(h.max()), "max_slot_load_after": int(after.max().item()),
           "mean_slot_load": round(float(h.mean()), 1)}
    print(json.dumps(rec), flush=True)


def _pct(sorted_vals, p: float) -> float:
    """Percentile of an ascending list (nearest rank)."""
    if not sorted_vals:
        return float("nan")
    i = min(len(sorted_vals) - 1, max(0, int(round(p / 100.0 * (len(sorted_vals) - 1)))))
    return sorted_vals[i]


def cpu_baseline(wl, n_slots: int):
    """The oracle (float64 NumPy) on a bounded sample: the whole front end for
    all tokens plus the expert work of the first ``n_slots`` local slots,
    scaled to the full layer by P_local / n_slots; BLAS on as many threads as
    the process may use (its CPU affinity), then the same on one thread over
    one slot."""
    from oracle import moe as om
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    d = wl.dims

    def run(slots):
        t0 = time.perf_counter()
        om.forward(wl, slots=range(slots))
        return time.perf_counter() - t0

    if threadpool_limits is not None:
        with threadpool_limits(limits=cores):
            blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            dt = run(n_slots)
    else:  # pragma: no cover
        blas, dt = 1, run(n_slots)
    est = dt * d.P_local / n_slots
    res = {"value": round(d.T / est, 3), "unit": "tokens/s", "cores": int(blas), "host_cores": cores,
           "kind": "oracle",
           "sample": f"oracle forward of {d.T} tokens with expert work on {n_slots} of {d.P_local} "
                     f"local slots ({dt:.1f}s), scaled x{d.P_local / n_slots:g} to all {d.P_local}; "
                     f"BLAS on {blas} threads of the {cores} cores this process may use"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            dt1 = run(1)
        res["single_thread"] = {"value": round(d.T / (dt1 * d.P_local), 3), "unit": "tokens/s",
                                "sample": f"the same with BLAS on one thread and expert work on 1 slot "
                                          f"({dt1:.1f}s), scaled x{d.P_local}"}
    return res


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, valid
    only while the GEMM sources are unchanged since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    e = t.get(f"{kernel}@{workload}")
    if not e or e.get("src_hash") != _src_hash(GEMM_SOURCES):
        return None
    return e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=3, help="weight copies rotated over steps")
    ap.add_argument("--workload", default="decode512", help=argparse.SUPPRESS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="leave out the 8192-token block")
    ap.add_argument("--cpu-slots", type=int, default=8)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: the token-count sweep and the EP-shaped prefill share, "
                         "one JSON line per point")
    ap.add_argument("--points", default=None,
                    help="with --sweep: comma-separated point names (sweep_T<T>, prefill_ep8_rank_share, eplb8192)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first copy a buffer of this many MiB with torch (a plain copy kernel of "
                         "known size, for scaling HBM byte counters under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported"}))
        sys.exit(2)

    if args.sweep:
        run_sweep(args.steps, args.warmup, args.copies,
                  None if args.points is None else set(args.points.split(",")))
        return
    import torch
    import synth
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        _log(f"[bench] calibration copies: 3 x {n} bytes read and written")
        del src, dst
    t0 = time.time()
    wl = synth.make(args.workload)
    _log(f"[bench] inputs for {args.workload} generated in {time.time() - t0:.1f}s")
    weights = packed_weights(wl, args.copies)
    r = measure(wl, weights, args.steps, args.warmup)
    d = r["d"]
    assert r["chosen"] == "small_m", r["chosen"]
    ms = r["wall"] * 1000.0 / args.steps
    value = d.T * args.steps / r["wall"]
    g1_bytes = w1_bytes(d, r["touched"])
    g1_gbs = g1_bytes / (r["gemm1_us"] * 1e-6) / 1e9
    g2_gbs = w2_bytes(d, r["touched"]) / (r["gemm2_us"] * 1e-6) / 1e9
    lay_bytes = layer_bytes(d, r["touched"])
    ev_ms = r["gpu_ms"] / args.steps
    lay_gbs = lay_bytes / (ev_ms * 1e-3) / 1e9
    line = {
        "metric": "MoE-layer tokens/s per GPU (512 & 8192 tok/rank); % HBM BW / MFMA peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x mxfp4 (f32 accumulate)",
        "data": "synthetic (seeded; random-init MXFP4 experts)",
        "config": {"workload": "decode share: T=512 tokens, d_model 7168, d_ff 2048, 384 experts, top-6 "
                               "sigmoid, 48 local experts, a8w4",
                   "T": d.T, "H": d.H, "F": d.F, "E": d.E, "k": d.k, "P_local": d.P_local,
                   "path": r["chosen"], "touched_slots": r["touched"], "rows": r["rows"],
                   "weight_copies": args.copies},
        # the dominant kernel: its algorithmic bytes are the W1 weights (MXFP4 +
        # scales) of the touched slots; its time is the average of the GEMM1
        # launches inside the timed forwards (HIP events around the launch)
        "roofline": {"bound": "hbm", "kernel": "k_gemm1_stream<true, 1, false>", "achieved": round(g1_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(g1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("k_gemm1_stream<true, 1, false>", args.workload),
                     "bytes_per_launch": g1_bytes, "avg_launch_us": round(r["gemm1_us"], 2)},
        "gemm2": {"kernel": "k_gemm2_stream<true, 1, false>", "bytes_per_launch": w2_bytes(d, r["touched"]),
                  "avg_launch_us": round(r["gemm2_us"], 2), "achieved": round(g2_gbs, 1),
                  "frac": round(g2_gbs / HBM_PEAK_GBS, 4)},
        "layer_roofline": {"bound": "hbm", "achieved": round(lay_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(lay_gbs / HBM_PEAK_GBS, 4), "bytes_per_step": lay_bytes,
                           "mfma_frac": round(layer_flops(d, r["rows"]) / (ev_ms * 1e-3) / 1e12 /
                                              FP8_PEAK_TFLOPS, 5),
                           "gpu_event_ms_per_step": round(ev_ms, 4)},
        "step_ms": {"median": round(_pct(r["per_step"], 50), 4), "p10": round(_pct(r["per_step"], 10), 4),
                    "p90": round(_pct(r["per_step"], 90), 4)},
    }
    line["layer_roofline"]["measured_copy_gbs"] = round(copy_rate_gbs(), 1)
    if not args.no_prefill:
        # the 8192-token half of the metric, on the same experts (weights reused)
        t0 = time.time()
        lit = synth.make("prefill8192", with_weights=False)
        rl = measure(lit, weights, args.steps, args.warmup)
        ep = synth.make_ep_shaped(8, with_weights=False)
        _log(f"[bench] prefill inputs generated in {time.time() - t0:.1f}s (timing included)")
        re_ = measure(ep, weights, args.steps, args.warmup, path="large_m")
        del ep, lit
        eps = summary(re_, "EP-shaped prefill share: 8 ranks x 8192 tokens routed into this GPU's 48 experts")
        eps["rank_share_tokens_per_s"] = round(8192 / (eps["ms_per_step"] * 1e-3), 1)
        eps["mfma_target"] = {"gemms_mfma_frac": 0.5, "met": eps["gemms_mfma_frac"] >= 0.5}
        line["prefill"] = {"literal_T8192": summary(rl, "prefill share: 8192 tokens into the 48 local experts"),
                           "ep8_T65536": eps}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_slots)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
