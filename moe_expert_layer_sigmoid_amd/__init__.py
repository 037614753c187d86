"""Python binding of libmoe, the gfx950 HIP library of one GPU's share of a
fused MoE expert layer (sigmoid top-k, EPLB remap + record, fp8 x MXFP4).

This module only marshals arguments: it checks dtypes and sizes of torch
tensors, reads their device pointers and the current HIP stream, and calls
the C ABI declared in ``include/moe.h`` by the same names.  Every step of the
layer runs in the library's kernels.  There is no fallback: if ``libmoe.so``
is missing or cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported size", -3: "workspace", -4: "hip",
          -5: "dims need more than the fixed scratch of moe_forward_noalloc"}
NOALLOC_SCRATCH_BYTES = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h
PATHS = {"auto": 0, "small_m": 1, "staged": 2, "large_m": 3}
PATH_NAMES = {v: k for k, v in PATHS.items()}

EXPORTS = ("moe_workspace_bytes", "moe_select_path", "moe_status_string", "moe_packed_bytes",
           "moe_pack_weights", "moe_route",
           "moe_eplb_remap_record", "moe_quant_permute", "moe_grouped_gemm1_swiglu",
           "moe_grouped_gemm2_combine", "moe_grouped_gemm1_swiglu_pairs", "moe_grouped_gemm2_combine_pairs",
           "moe_forward", "moe_eplb_rebalance", "moe_eplb_migrate",
           "moe_router_workspace_bytes", "moe_router_logits", "moe_forward_small_m",
           "moe_a16w4_workspace_bytes", "moe_forward_a16w4", "moe_forward_noalloc", "moe_replica_of")


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed with status {code} ({STATUS.get(code, 'unknown')})")
        self.code = code


class Dims(ctypes.Structure):
    """moe_dims_t"""
    _fields_ = [("T", ctypes.c_int32), ("T_max", ctypes.c_int32), ("H", ctypes.c_int32),
                ("F", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("P_total", ctypes.c_int32), ("p0", ctypes.c_int32), ("P_local", ctypes.c_int32),
                ("R_max", ctypes.c_int32), ("token_id_base", ctypes.c_uint32),
                ("small_m_max", ctypes.c_int32), ("large_m_min", ctypes.c_int32)]

    @classmethod
    def of(cls, d, **kw) -> "Dims":
        """From any object with the same attribute names (e.g. synth.Dims)."""
        vals = {f: getattr(d, f, 0) for f, _ in cls._fields_}
        vals.update(kw)
        return cls(**{k: int(v) for k, v in vals.items()})


class Taps(ctypes.Structure):
    """moe_taps_t"""
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_ids", "topk_w", "phys_ids", "counts", "offsets",
                                                "row_of_pair", "pair_of_row", "xq", "xs", "aq", "as_",
                                                "xq_tok", "xs_tok", "aq_pair", "as_pair")]
    _fields_ += [("gemm1_events", ctypes.c_void_p * 2), ("gemm2_events", ctypes.c_void_p * 2)]


def _event_handle(ev) -> int:
    """The hipEvent_t behind a torch.cuda.Event (torch creates it at the first record)."""
    if ev.cuda_event == 0:
        ev.record()
    return ev.cuda_event


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it was not built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m moe_expert_layer_sigmoid_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(Dims)
        I = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [D]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_select_path.argtypes = [D]
        L.moe_select_path.restype = I
        L.moe_status_string.argtypes = [I]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_packed_bytes.argtypes = [D, I]
        L.moe_packed_bytes.restype = ctypes.c_size_t
        L.moe_pack_weights.argtypes = [D, P, P, P, P, P, P, P, P, P]
        L.moe_route.argtypes = [D, P, P, P, P]
        L.moe_eplb_remap_record.argtypes = [D, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_quant_permute.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_grouped_gemm1_swiglu.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_grouped_gemm2_combine.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_grouped_gemm1_swiglu_pairs.argtypes = [D, P, P, P, P, P, P, P, P, P]
        L.moe_grouped_gemm2_combine_pairs.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_forward.argtypes = [D, I, P, P, P, P, P, P, P, P, P, P, ctypes.POINTER(Taps),
                                  ctypes.POINTER(ctypes.c_int), P, ctypes.c_size_t, P]
        L.moe_forward_small_m.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, ctypes.POINTER(Taps), P,
                                          ctypes.c_size_t, P]
        L.moe_forward_small_m.restype = I
        L.moe_forward_noalloc.argtypes = [D, I, P, P, P, P, P, P, P, P, P, P, ctypes.POINTER(ctypes.c_int), P]
        L.moe_forward_noalloc.restype = I
        L.moe_a16w4_workspace_bytes.argtypes = [D]
        L.moe_a16w4_workspace_bytes.restype = ctypes.c_size_t
        L.moe_forward_a16w4.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.POINTER(Taps), P, P,
                                        ctypes.c_size_t, P]
        L.moe_forward_a16w4.restype = I
        L.moe_router_workspace_bytes.argtypes = [D]
        L.moe_router_workspace_bytes.restype = ctypes.c_size_t
        L.moe_router_logits.argtypes = [D, P, P, P, P, ctypes.c_size_t, P]
        L.moe_router_logits.restype = I
        L.moe_replica_of.argtypes = [ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32]
        L.moe_replica_of.restype = ctypes.c_int32
        L.moe_eplb_rebalance.argtypes = [I, I, I, I, P, P, P, P, P]
        L.moe_eplb_migrate.argtypes = [D, P, I, P, P, P, P, P, P, P, P, P]
        for n in ("moe_pack_weights", "moe_route", "moe_eplb_remap_record", "moe_quant_permute",
                  "moe_grouped_gemm1_swiglu", "moe_grouped_gemm2_combine", "moe_grouped_gemm1_swiglu_pairs",
                  "moe_grouped_gemm2_combine_pairs", "moe_forward", "moe_eplb_rebalance", "moe_eplb_migrate"):
            getattr(L, n).restype = I
        _lib_handle = L
    return _lib_handle


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel_min: int = 0):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() < numel_min:
        raise ValueError(f"{name}: {t.numel()} elements, need at least {numel_min}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


u8, i32, f32, i16 = torch.uint8, torch.int32, torch.float32, torch.int16


def _bf16(t: torch.Tensor) -> torch.dtype:
    return t.dtype if t.dtype in (torch.bfloat16, torch.int16, torch.uint16) else torch.bfloat16


def _sizes(d: Dims):
    TK, TMK = d.T * d.k, d.T_max * d.k
    return TK, TMK


# ----------------------------------------------------------------------------
# the C ABI, same names
# ----------------------------------------------------------------------------

def moe_workspace_bytes(d: Dims) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(d)))


def moe_select_path(d: Dims) -> str:
    return PATH_NAMES[int(lib().moe_select_path(ctypes.byref(d)))]


def moe_status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def moe_replica_of(token_id: int, rep_count: int, R_max: int) -> int:
    return int(lib().moe_replica_of(int(token_id) & 0xFFFFFFFF, int(rep_count), int(R_max)))


def moe_packed_bytes(d: Dims, which: int) -> int:
    return int(lib().moe_packed_bytes(ctypes.byref(d), int(which)))


def moe_pack_weights(d: Dims, w1, w1s, w2, w2s, pw1, pw1s, pw2, pw2s, stream=None):
    nw1, ns1 = d.P_local * 2 * d.F * d.H // 2, d.P_local * 2 * d.F * d.H // 32
    nw2, ns2 = d.P_local * d.H * d.F // 2, d.P_local * d.H * d.F // 32
    rc = lib().moe_pack_weights(
        ctypes.byref(d), _ptr(w1, "w1", u8, nw1), _ptr(w1s, "w1s", u8, ns1), _ptr(w2, "w2", u8, nw2),
        _ptr(w2s, "w2s", u8, ns2), _ptr(pw1, "pw1", u8, moe_packed_bytes(d, 0)),
        _ptr(pw1s, "pw1s", u8, moe_packed_bytes(d, 1)), _ptr(pw2, "pw2", u8, moe_packed_bytes(d, 2)),
        _ptr(pw2s, "pw2s", u8, moe_packed_bytes(d, 3)), _stream(stream))
    _check("moe_pack_weights", rc)


def pack_weights(d: Dims, w1, w1s, w2, w2s, stream=None):
    """Allocate and fill the packed weight buffers; returns (pw1, pw1s, pw2, pw2s)."""
    dev = w1.device
    out = tuple(torch.empty(moe_packed_bytes(d, i), dtype=u8, device=dev) for i in range(4))
    moe_pack_weights(d, w1, w1s, w2, w2s, *out, stream=stream)
    return out


def workspace(d: Dims, device="cuda") -> torch.Tensor:
    """A workspace of moe_workspace_bytes(d) bytes (torch-allocated, 256-B aligned)."""
    n = moe_workspace_bytes(d)
    return torch.empty(max(n, 256), dtype=u8, device=device)


def moe_route(d: Dims, logits, topk_ids, topk_w, stream=None):
    TK, _ = _sizes(d)
    rc = lib().moe_route(ctypes.byref(d), _ptr(logits, "logits", f32, d.T * d.E),
                         _ptr(topk_ids, "topk_ids", i32, TK), _ptr(topk_w, "topk_w", f32, TK), _stream(stream))
    _check("moe_route", rc)


def moe_eplb_remap_record(d: Dims, topk_ids, rep_count, rep_slots, phys_ids, load_hist, ws, stream=None):
    TK, _ = _sizes(d)
    rc = lib().moe_eplb_remap_record(
        ctypes.byref(d), _ptr(topk_ids, "topk_ids", i32, TK), _ptr(rep_count, "rep_count", i32, d.E),
        _ptr(rep_slots, "rep_slots", i32, d.E * d.R_max), _ptr(phys_ids, "phys_ids", i32, TK),
        _ptr(load_hist, "load_hist", i32, d.P_total), _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_eplb_remap_record", rc)


def moe_quant_permute(d: Dims, x, phys_ids, xq, xs, counts, offsets, row_of_pair, pair_of_row, ws, stream=None):
    TK, TMK = _sizes(d)
    rc = lib().moe_quant_permute(
        ctypes.byref(d), _ptr(x, "x", _bf16(x), d.T * d.H), _ptr(phys_ids, "phys_ids", i32, TK),
        _ptr(xq, "xq", u8, TMK * d.H), _ptr(xs, "xs", u8, TMK * (d.H // 128)),
        _ptr(counts, "counts", i32, d.P_local), _ptr(offsets, "offsets", i32, d.P_local + 1),
        _ptr(row_of_pair, "row_of_pair", i32, TK), _ptr(pair_of_row, "pair_of_row", i32, TMK),
        _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_quant_permute", rc)


def moe_grouped_gemm1_swiglu(d: Dims, xq, xs, offsets, pw1, pw1s, aq, as_, ws, stream=None):
    _, TMK = _sizes(d)
    rc = lib().moe_grouped_gemm1_swiglu(
        ctypes.byref(d), _ptr(xq, "xq", u8, TMK * d.H), _ptr(xs, "xs", u8, TMK * (d.H // 128)),
        _ptr(offsets, "offsets", i32, d.P_local + 1),
        _ptr(pw1, "pw1", u8, moe_packed_bytes(d, 0)), _ptr(pw1s, "pw1s", u8, moe_packed_bytes(d, 1)),
        _ptr(aq, "aq", u8, TMK * d.F), _ptr(as_, "as", u8, TMK * (d.F // 128)),
        _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_grouped_gemm1_swiglu", rc)


def moe_grouped_gemm2_combine(d: Dims, aq, as_, offsets, pw2, pw2s, row_of_pair, topk_w, out, ws, stream=None):
    TK, TMK = _sizes(d)
    rc = lib().moe_grouped_gemm2_combine(
        ctypes.byref(d), _ptr(aq, "aq", u8, TMK * d.F), _ptr(as_, "as", u8, TMK * (d.F // 128)),
        _ptr(offsets, "offsets", i32, d.P_local + 1),
        _ptr(pw2, "pw2", u8, moe_packed_bytes(d, 2)), _ptr(pw2s, "pw2s", u8, moe_packed_bytes(d, 3)),
        _ptr(row_of_pair, "row_of_pair", i32, TK), _ptr(topk_w, "topk_w", f32, TK),
        _ptr(out, "out", _bf16(out), d.T * d.H), _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_grouped_gemm2_combine", rc)


def moe_grouped_gemm1_swiglu_pairs(d: Dims, xq_tok, xs_tok, phys_ids, pw1, pw1s, aq_pair, as_pair, counts,
                                   stream=None):
    TK = d.T * d.k
    rc = lib().moe_grouped_gemm1_swiglu_pairs(
        ctypes.byref(d), _ptr(xq_tok, "xq_tok", u8, d.T * d.H), _ptr(xs_tok, "xs_tok", u8, d.T * (d.H // 128)),
        _ptr(phys_ids, "phys_ids", i32, TK),
        _ptr(pw1, "pw1", u8, moe_packed_bytes(d, 0)), _ptr(pw1s, "pw1s", u8, moe_packed_bytes(d, 1)),
        _ptr(aq_pair, "aq_pair", u8, TK * d.F), _ptr(as_pair, "as_pair", u8, TK * (d.F // 128)),
        _ptr(counts, "counts", i32, d.P_local), _stream(stream))
    _check("moe_grouped_gemm1_swiglu_pairs", rc)


def moe_grouped_gemm2_combine_pairs(d: Dims, aq_pair, as_pair, phys_ids, pw2, pw2s, topk_w, counts, offsets, out, ws,
                                    stream=None):
    TK = d.T * d.k
    rc = lib().moe_grouped_gemm2_combine_pairs(
        ctypes.byref(d), _ptr(aq_pair, "aq_pair", u8, TK * d.F), _ptr(as_pair, "as_pair", u8, TK * (d.F // 128)),
        _ptr(phys_ids, "phys_ids", i32, TK),
        _ptr(pw2, "pw2", u8, moe_packed_bytes(d, 2)), _ptr(pw2s, "pw2s", u8, moe_packed_bytes(d, 3)),
        _ptr(topk_w, "topk_w", f32, TK), _ptr(counts, "counts", i32, d.P_local),
        _ptr(offsets, "offsets", i32, d.P_local + 1), _ptr(out, "out", _bf16(out), d.T * d.H),
        _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_grouped_gemm2_combine_pairs", rc)


def make_taps(d: Dims, device="cuda") -> Dict[str, torch.Tensor]:
    """Device buffers for every tap of moe_forward."""
    TK, TMK = _sizes(d)
    z = lambda n, dt: torch.zeros(max(n, 1), dtype=dt, device=device)  # noqa: E731
    return dict(topk_ids=z(TK, i32), topk_w=z(TK, f32), phys_ids=z(TK, i32), counts=z(d.P_local, i32),
                offsets=z(d.P_local + 1, i32), row_of_pair=z(TK, i32), pair_of_row=z(TMK, i32),
                xq=z(TMK * d.H, u8), xs=z(TMK * (d.H // 128), u8), aq=z(TMK * d.F, u8),
                as_=z(TMK * (d.F // 128), u8), xq_tok=z(d.T * d.H, u8), xs_tok=z(d.T * (d.H // 128), u8),
                aq_pair=z(TK * d.F, u8), as_pair=z(TK * (d.F // 128), u8))


def moe_forward(d: Dims, x, logits, pw1, pw1s, pw2, pw2s, rep_count, rep_slots, out, ws, load_hist=None,
                path: str = "auto", taps: Optional[Dict[str, torch.Tensor]] = None, stream=None,
                gemm_events=None) -> str:
    """Run the whole layer on packed weights; returns the path taken
    ("small_m", "staged", "large_m").  ``gemm_events`` (optional): four
    torch.cuda.Event recorded around the GEMM1 and the GEMM2 launch
    (begin1, end1, begin2, end2)."""
    TK, TMK = _sizes(d)
    tp = None
    if taps is not None:
        need = dict(topk_ids=(i32, TK), topk_w=(f32, TK), phys_ids=(i32, TK), counts=(i32, d.P_local),
                    offsets=(i32, d.P_local + 1), row_of_pair=(i32, TK), pair_of_row=(i32, TMK),
                    xq=(u8, TMK * d.H), xs=(u8, TMK * (d.H // 128)), aq=(u8, TMK * d.F),
                    as_=(u8, TMK * (d.F // 128)), xq_tok=(u8, d.T * d.H), xs_tok=(u8, d.T * (d.H // 128)),
                    aq_pair=(u8, TK * d.F), as_pair=(u8, TK * (d.F // 128)))
        tp = Taps(**{n: _ptr(taps.get(n), n, *need[n]) for n in need})
    if gemm_events is not None:
        tp = tp if tp is not None else Taps()
        h = [_event_handle(e) for e in gemm_events]
        tp.gemm1_events[0], tp.gemm1_events[1], tp.gemm2_events[0], tp.gemm2_events[1] = h
    chosen = ctypes.c_int(-1)
    rc = lib().moe_forward(
        ctypes.byref(d), PATHS[path], _ptr(x, "x", _bf16(x), d.T * d.H), _ptr(logits, "logits", f32, d.T * d.E),
        _ptr(pw1, "pw1", u8, moe_packed_bytes(d, 0)), _ptr(pw1s, "pw1s", u8, moe_packed_bytes(d, 1)),
        _ptr(pw2, "pw2", u8, moe_packed_bytes(d, 2)), _ptr(pw2s, "pw2s", u8, moe_packed_bytes(d, 3)),
        _ptr(rep_count, "rep_count", i32, d.E), _ptr(rep_slots, "rep_slots", i32, d.E * d.R_max),
        _ptr(load_hist, "load_hist", i32, d.P_total), _ptr(out, "out", _bf16(out), d.T * d.H),
        ctypes.byref(tp) if tp is not None else None, ctypes.byref(chosen),
        _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_forward", rc)
    return PATH_NAMES[chosen.value]


def moe_forward_noalloc(d: Dims, x, logits, pw1, pw1s, pw2, pw2s, rep_count, rep_slots, out, load_hist=None,
                        path: str = "auto", stream=None) -> str:
    """moe_forward without a workspace: the library's fixed per-GPU scratch
    (NOALLOC_SCRATCH_BYTES) serves instead, so the call allocates nothing.
    Calls that overlap in time on one GPU share that scratch and race.
    Returns the path taken."""
    chosen = ctypes.c_int(-1)
    rc = lib().moe_forward_noalloc(
        ctypes.byref(d), PATHS[path], _ptr(x, "x", _bf16(x), d.T * d.H), _ptr(logits, "logits", f32, d.T * d.E),
        _ptr(pw1, "pw1", u8, moe_packed_bytes(d, 0)), _ptr(pw1s, "pw1s", u8, moe_packed_bytes(d, 1)),
        _ptr(pw2, "pw2", u8, moe_packed_bytes(d, 2)), _ptr(pw2s, "pw2s", u8, moe_packed_bytes(d, 3)),
        _ptr(rep_count, "rep_count", i32, d.E), _ptr(rep_slots, "rep_slots", i32, d.E * d.R_max),
        _ptr(load_hist, "load_hist", i32, d.P_total), _ptr(out, "out", _bf16(out), d.T * d.H),
        ctypes.byref(chosen), _stream(stream))
    _check("moe_forward_noalloc", rc)
    return PATH_NAMES[chosen.value]


def moe_forward_small_m(d: Dims, num_tokens, x, logits, pw1, pw1s, pw2, pw2s, rep_count, rep_slots, out, ws,
                        load_hist=None, taps: Optional[Dict[str, torch.Tensor]] = None, stream=None) -> None:
    """The small-input path with the valid token count read on the device
    from ``num_tokens`` (int32 device tensor, one element); d.T is the bucket
    capacity.  Allocates nothing: safe inside torch.cuda.graph capture."""
    TK, _ = _sizes(d)
    tp = None
    if taps is not None:
        need = dict(topk_ids=(i32, TK), topk_w=(f32, TK), phys_ids=(i32, TK), counts=(i32, d.P_local),
                    offsets=(i32, d.P_local + 1), xq_tok=(u8, d.T * d.H), xs_tok=(u8, d.T * (d.H // 128)),
                    aq_pair=(u8, TK * d.F), as_pair=(u8, TK * (d.F // 128)))
        tp = Taps(**{n: _ptr(taps.get(n), n, *need[n]) for n in need})
    rc = lib().moe_forward_small_m(
        ctypes.byref(d), _ptr(num_tokens, "num_tokens", i32, 1), _ptr(x, "x", _bf16(x), d.T * d.H),
        _ptr(logits, "logits", f32, d.T * d.E),
        _ptr(pw1, "pw1", u8, moe_packed_bytes(d, 0)), _ptr(pw1s, "pw1s", u8, moe_packed_bytes(d, 1)),
        _ptr(pw2, "pw2", u8, moe_packed_bytes(d, 2)), _ptr(pw2s, "pw2s", u8, moe_packed_bytes(d, 3)),
        _ptr(rep_count, "rep_count", i32, d.E), _ptr(rep_slots, "rep_slots", i32, d.E * d.R_max),
        _ptr(load_hist, "load_hist", i32, d.P_total), _ptr(out, "out", _bf16(out), d.T * d.H),
        ctypes.byref(tp) if tp is not None else None, _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_forward_small_m", rc)


# ----------------------------------------------------------------------------
# EPLB rebalance (host) and weight migration (device)
# ----------------------------------------------------------------------------

def _host_i32(a, name: str, n: int):
    import numpy as np
    if isinstance(a, torch.Tensor):
        if a.device.type != "cpu":
            raise ValueError(f"{name}: must be a host array")
        a = a.numpy()
    a = np.ascontiguousarray(a, dtype=np.int32)
    if a.size != n:
        raise ValueError(f"{name}: {a.size} elements, expected {n}")
    return a


def moe_eplb_rebalance(E: int, P_total: int, n_ranks: int, R_max: int, load_hist, slot_expert_old):
    """New replica table from recorded slot loads (host arrays in and out).
    Returns numpy int32 (rep_count [E], rep_slots [E, R_max], slot_expert_new [P_total])."""
    import numpy as np
    h = _host_i32(load_hist, "load_hist", P_total)
    old = _host_i32(slot_expert_old, "slot_expert_old", P_total)
    rc = np.zeros(E, np.int32)
    rs = np.zeros((E, R_max), np.int32)
    new = np.zeros(P_total, np.int32)
    c = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    st = lib().moe_eplb_rebalance(int(E), int(P_total), int(n_ranks), int(R_max), c(h), c(old), c(rc), c(rs), c(new))
    _check("moe_eplb_rebalance", st)
    return rc, rs, new


def moe_eplb_migrate(d: Dims, src_expert, n_pool: int, pool, slots, stream=None):
    """Copy pool experts into local slots: ``pool`` and ``slots`` are packed
    weight tuples (pw1, pw1s, pw2, pw2s) over n_pool experts and d.P_local
    slots; src_expert i32 [P_local] on the device (-1 = keep)."""
    per = [moe_packed_bytes(d, i) // d.P_local for i in range(4)]
    names = ("pw1", "pw1s", "pw2", "pw2s")
    pp = [_ptr(t, "pool_" + n, u8, per[i] * n_pool) for i, (t, n) in enumerate(zip(pool, names))]
    sp = [_ptr(t, n, u8, per[i] * d.P_local) for i, (t, n) in enumerate(zip(slots, names))]
    rc = lib().moe_eplb_migrate(ctypes.byref(d), _ptr(src_expert, "src_expert", i32, d.P_local), int(n_pool),
                                *pp, *sp, _stream(stream))
    _check("moe_eplb_migrate", rc)


# ----------------------------------------------------------------------------
# Router projection
# ----------------------------------------------------------------------------

def moe_router_workspace_bytes(d: Dims) -> int:
    return int(lib().moe_router_workspace_bytes(ctypes.byref(d)))


def router_workspace(d: Dims, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_router_workspace_bytes(d), 256), dtype=u8, device=device)


def moe_router_logits(d: Dims, x, w_gate, logits, ws, stream=None):
    """logits f32 [T, E] = x bf16 [T, H] (int16 bits or bfloat16) times w_gate bf16 [E, H] transposed."""
    rc = lib().moe_router_logits(ctypes.byref(d), _ptr(x, "x", _bf16(x), d.T * d.H),
                                 _ptr(w_gate, "w_gate", _bf16(w_gate), d.E * d.H),
                                 _ptr(logits, "logits", f32, d.T * d.E), _ptr(ws, "workspace", u8), ws.numel(),
                                 _stream(stream))
    _check("moe_router_logits", rc)


# ----------------------------------------------------------------------------
# a16w4 variant
# ----------------------------------------------------------------------------

def moe_a16w4_workspace_bytes(d: Dims) -> int:
    return int(lib().moe_a16w4_workspace_bytes(ctypes.byref(d)))


def a16w4_workspace(d: Dims, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_a16w4_workspace_bytes(d), 256), dtype=u8, device=device)


def moe_forward_a16w4(d: Dims, x, logits, pw1, pw1s, pw2, pw2s, rep_count, rep_slots, out, ws, load_hist=None,
                      taps: Optional[Dict[str, torch.Tensor]] = None, act=None, stream=None) -> None:
    """The layer with bf16 activations on the packed MXFP4 experts.  ``act``
    (optional, bf16 [T_max*k, F] as int16 bits) receives the GEMM1 act rows."""
    TK, TMK = _sizes(d)
    tp = None
    if taps is not None:
        need = dict(topk_ids=(i32, TK), topk_w=(f32, TK), phys_ids=(i32, TK), counts=(i32, d.P_local),
                    offsets=(i32, d.P_local + 1), row_of_pair=(i32, TK), pair_of_row=(i32, TMK))
        tp = Taps(**{n: _ptr(taps.get(n), n, *need[n]) for n in need})
    rc = lib().moe_forward_a16w4(
        ctypes.byref(d), _ptr(x, "x", _bf16(x), d.T * d.H), _ptr(logits, "logits", f32, d.T * d.E),
        _ptr(pw1, "pw1", u8, moe_packed_bytes(d, 0)), _ptr(pw1s, "pw1s", u8, moe_packed_bytes(d, 1)),
        _ptr(pw2, "pw2", u8, moe_packed_bytes(d, 2)), _ptr(pw2s, "pw2s", u8, moe_packed_bytes(d, 3)),
        _ptr(rep_count, "rep_count", i32, d.E), _ptr(rep_slots, "rep_slots", i32, d.E * d.R_max),
        _ptr(load_hist, "load_hist", i32, d.P_total), _ptr(out, "out", _bf16(out), d.T * d.H),
        ctypes.byref(tp) if tp is not None else None,
        _ptr(act, "act", _bf16(act), TMK * d.F) if act is not None else None,
        _ptr(ws, "workspace", u8), ws.numel(), _stream(stream))
    _check("moe_forward_a16w4", rc)
