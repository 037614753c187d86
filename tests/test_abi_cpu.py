"""The C-ABI library loads on the CPU, exports every declared symbol, and
rejects bad arguments on the host before any launch (no GPU needed)."""

import ctypes
import os
import re

import pytest

import moe_expert_layer_sigmoid_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(mx.LIB_PATH), reason="libmoe.so not built")


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(moe_\w+)\s*\(", txt))
    return names


def test_exports_every_declared_symbol():
    decl = _declared()
    assert set(mx.EXPORTS) <= decl
    L = mx.lib()
    for n in sorted(decl):
        assert hasattr(L, n), n


def _dims(**kw):
    base = dict(T=512, T_max=512, H=7168, F=2048, E=384, k=6, P_total=384, p0=0, P_local=48, R_max=1)
    base.update(kw)
    return mx.Dims(**base)


def test_workspace_bytes_and_invalid_dims():
    d = _dims()
    n = mx.moe_workspace_bytes(d)
    rows = 512 * 6
    assert n >= rows * (7168 + 56 + 2048 + 16 + 7168 * 4)
    assert mx.moe_workspace_bytes(_dims(T=8192, T_max=8192)) > n
    for bad in (dict(T=513), dict(H=100), dict(F=0), dict(k=0), dict(k=17), dict(E=2000),
                dict(P_local=0), dict(p0=340), dict(R_max=0), dict(P_total=2000), dict(T=-1)):
        assert mx.moe_workspace_bytes(_dims(**bad)) == 0, bad
    # depends on T_max only
    assert mx.moe_workspace_bytes(_dims(T=1)) == n


def test_select_path_thresholds():
    assert mx.moe_select_path(_dims(T=1)) == "small_m"
    assert mx.moe_select_path(_dims(T=512)) == "small_m"
    assert mx.moe_select_path(_dims(T=513, T_max=8192)) == "staged"
    assert mx.moe_select_path(_dims(T=1023, T_max=8192)) == "staged"
    assert mx.moe_select_path(_dims(T=1024, T_max=8192)) == "large_m"
    assert mx.moe_select_path(_dims(T=100, small_m_max=64, large_m_min=100)) == "large_m"
    assert mx.moe_select_path(_dims(T=64, small_m_max=64)) == "small_m"
    # the small-input path lists each slot's pairs in one block: at most 1024 tokens
    assert mx.moe_select_path(_dims(T=1024, T_max=8192, small_m_max=4096, large_m_min=8192)) == "small_m"
    assert mx.moe_select_path(_dims(T=1025, T_max=8192, small_m_max=4096, large_m_min=8192)) == "staged"


def test_status_strings():
    for c in (0, -1, -2, -3, -4, -5, 7):
        assert mx.moe_status_string(c)


def _forward_raw(d, ptrs, ws, ws_bytes, path=0):
    L = mx.lib()
    chosen = ctypes.c_int(-1)
    P = ctypes.c_void_p
    rc = L.moe_forward(ctypes.byref(d), path, *[P(p) if p else None for p in ptrs], None,
                       ctypes.byref(chosen), P(ws) if ws else None, ws_bytes, None)
    return rc, chosen.value


GOOD = [0x1000 * (i + 1) for i in range(10)]  # aligned fake device addresses, never dereferenced


def test_host_validation_before_launch():
    d = _dims()
    need = mx.moe_workspace_bytes(d)
    # null required pointer
    p = list(GOOD)
    p[0] = 0
    assert _forward_raw(d, p, 0x100000, need)[0] == -1
    # misaligned pointer
    p = list(GOOD)
    p[3] = 0x1008
    assert _forward_raw(d, p, 0x100000, need)[0] == -1
    # workspace missing / too small
    assert _forward_raw(d, GOOD, 0, 0)[0] == -3
    assert _forward_raw(d, GOOD, 0x100000, need - 1)[0] == -3
    # T > T_max, k mismatch analog, unsupported sizes
    assert _forward_raw(_dims(T=600), GOOD, 0x100000, need)[0] == -1
    assert _forward_raw(_dims(k=17), GOOD, 0x100000, need)[0] == -2
    assert _forward_raw(_dims(H=200), GOOD, 0x100000, need)[0] == -1
    # bad path
    assert _forward_raw(d, GOOD, 0x100000, need, path=9)[0] == -1
    # the small-input path beyond 1024 tokens is refused, not rerouted
    big = _dims(T=1025, T_max=1025)
    assert _forward_raw(big, GOOD, 0x100000, mx.moe_workspace_bytes(big), path=1)[0] == -2
    # widths beyond 16384 are refused; the large-input path's tiled GEMMs stop
    # at 8192 (their LDS), and AUTO then takes the staged path
    assert _forward_raw(_dims(H=16512), GOOD, 0x100000, need)[0] == -2
    wide = _dims(T=2048, T_max=2048, H=16384)
    wneed = mx.moe_workspace_bytes(wide)
    assert _forward_raw(wide, GOOD, 0x100000, wneed, path=3)[0] == -2
    assert mx.moe_select_path(wide) == "staged"


def test_zero_tokens_is_a_no_op():
    d = _dims(T=0)
    need = mx.moe_workspace_bytes(d)
    rc, chosen = _forward_raw(d, GOOD, 0x100000, need)
    assert rc == 0 and chosen == 1  # small-M, nothing launched
    L = mx.lib()
    P = ctypes.c_void_p
    assert L.moe_route(ctypes.byref(d), P(0x1000), P(0x2000), P(0x3000), None) == 0
    assert L.moe_route(ctypes.byref(d), None, P(0x2000), P(0x3000), None) == -1


def test_next_row_entry_points_validate_on_the_host():
    """Router projection, graph-bucket forward, a16w4 forward and EPLB
    migration: argument errors come back before any launch; zero tokens
    launch nothing."""
    L = mx.lib()
    P = ctypes.c_void_p
    d = _dims()
    G = [P(a) for a in GOOD]
    # router projection
    rb = mx.moe_router_workspace_bytes(d)
    assert rb > 0 and mx.moe_router_workspace_bytes(_dims(T_max=8192)) > rb
    assert L.moe_router_logits(ctypes.byref(d), G[0], G[1], G[2], G[3], rb - 1, None) == -3
    assert L.moe_router_logits(ctypes.byref(d), None, G[1], G[2], G[3], rb, None) == -1
    assert L.moe_router_logits(ctypes.byref(d), G[0], G[1], P(0x2004), G[3], rb, None) == -1
    z = _dims(T=0)
    assert L.moe_router_logits(ctypes.byref(z), G[0], G[1], G[2], G[3], mx.moe_router_workspace_bytes(z), None) == 0

    # graph-bucket small-input forward
    need = mx.moe_workspace_bytes(d)
    args = G[:10]
    assert L.moe_forward_small_m(ctypes.byref(d), None, *args, None, P(0x100000), need, None) == -1
    assert L.moe_forward_small_m(ctypes.byref(d), P(0x1002), *args, None, P(0x100000), need, None) == -1
    big = _dims(T=1025, T_max=1025)
    assert L.moe_forward_small_m(ctypes.byref(big), P(0x1000), *args, None, P(0x100000),
                                 mx.moe_workspace_bytes(big), None) == -2
    assert L.moe_forward_small_m(ctypes.byref(z), P(0x1000), *args, None, P(0x100000),
                                 mx.moe_workspace_bytes(z), None) == 0

    # a16w4 forward
    ab = mx.moe_a16w4_workspace_bytes(d)
    assert ab > need
    assert L.moe_forward_a16w4(ctypes.byref(d), *args, None, None, P(0x100000), ab - 1, None) == -3
    bad = list(args)
    bad[2] = None
    assert L.moe_forward_a16w4(ctypes.byref(d), *bad, None, None, P(0x100000), ab, None) == -1
    huge = _dims(T=1, T_max=1 << 20, H=16384)
    # size queries are size_t through the binding (no 32-bit truncation)
    assert mx.moe_a16w4_workspace_bytes(huge) > 2 ** 32 and mx.moe_workspace_bytes(huge) > 2 ** 32
    assert L.moe_forward_a16w4(ctypes.byref(huge), *args, None, None, P(0x100000),
                               mx.moe_a16w4_workspace_bytes(huge), None) == -2
    assert L.moe_forward_a16w4(ctypes.byref(z), *args, None, None, P(0x100000),
                               mx.moe_a16w4_workspace_bytes(z), None) == 0

    # EPLB migration (a valid call would launch: only errors here)
    assert L.moe_eplb_migrate(ctypes.byref(d), G[0], 0, *G[1:9], None) == -1
    assert L.moe_eplb_migrate(ctypes.byref(d), G[0], 384, P(0x1001), *G[2:9], None) == -1
    assert L.moe_eplb_migrate(ctypes.byref(_dims(H=100)), G[0], 384, *G[1:9], None) == -1


def test_noalloc_entry_validates_on_the_host():
    """moe_forward_noalloc refuses dims beyond its fixed scratch (and bad dims)
    before it touches the GPU; the scratch size matches the header's."""
    L = mx.lib()
    P = ctypes.c_void_p
    G = [P(a) for a in GOOD]
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == mx.NOALLOC_SCRATCH_BYTES
    # the stated capacity at d_model 7168, d_ff 2048, top-6
    assert mx.moe_workspace_bytes(_dims(T=1, T_max=587)) <= mx.NOALLOC_SCRATCH_BYTES
    assert mx.moe_workspace_bytes(_dims(T=1, T_max=588)) > mx.NOALLOC_SCRATCH_BYTES
    chosen = ctypes.c_int(-1)
    call = lambda d: L.moe_forward_noalloc(ctypes.byref(d), 0, *G[:10], ctypes.byref(chosen), None)  # noqa: E731
    assert call(_dims(T=1, T_max=588)) == -5
    assert call(_dims(T=8192, T_max=8192)) == -5
    assert call(_dims(k=17)) == -2
    assert call(_dims(T=600)) == -1
    assert chosen.value == -1  # nothing chosen, nothing launched
    assert "scratch" in mx.moe_status_string(-5)


def test_replica_index_and_its_guard():
    """The remap's replica rule on the host (the kernels use the same
    function): fmix32(token id) mod rep_count, against the oracle's hash, and a
    rep_count outside [1, R_max] clamped so the index stays in the table row."""
    import numpy as np
    from oracle import moe as om
    ids = np.array([0, 1, 2, 12345, 2 ** 31 - 1, 2 ** 32 - 1, 987654321], np.uint64)
    h = om.fmix32(ids).astype(np.int64)
    for count in (1, 2, 3, 7, 64):
        got = [mx.moe_replica_of(int(t), count, 64) for t in ids]
        assert got == list(h % count)
    for bad, R_max in ((0, 4), (-5, 4), (9, 4), (1000, 64)):
        for t in ids:
            r = mx.moe_replica_of(int(t), bad, R_max)
            assert 0 <= r < R_max
            assert r == int(om.fmix32(np.array([t], np.uint64))[0]) % min(max(bad, 1), R_max)
