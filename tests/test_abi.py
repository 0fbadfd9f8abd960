"""The C-ABI library on the host: it loads, exports every declared symbol, and rejects
invalid calls with the documented status before any HIP call (so these run without a
GPU)."""
import ctypes
import os
import re
from ctypes import POINTER, byref, c_int32, c_size_t, c_void_p

import numpy as np
import pytest

import graphgen as gg
from sparse_graph_attention_02_amd import capi
from sparse_graph_attention_02_amd import Plan, default_opts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "graph_attn.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(graph_attn_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(capi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    # and the binding wraps exactly the declared surface
    assert sorted(capi.exported_names()) == names


def test_version_and_status_strings():
    assert capi.graph_attn_version().decode().startswith("graph_attn")
    for s in range(9):
        assert capi.lib().graph_attn_status_string(s).decode().startswith("GA_")
    assert capi.lib().graph_attn_status_string(99) == b"unknown ga_status"


def _create(ip, ix, opts=None):
    h = c_void_p()
    st = capi.raw_status("graph_attn_plan_create",
                         np.ascontiguousarray(ip, np.int32).ctypes.data_as(POINTER(c_int32)),
                         np.ascontiguousarray(ix, np.int32).ctypes.data_as(POINTER(c_int32)),
                         len(ip) - 1, len(ix), byref(opts) if opts else None, byref(h))
    return st, h


@pytest.mark.parametrize("ip,ix", [
    ([1, 2, 3], [0, 1, 1]),          # indptr[0] != 0
    ([0, 3, 2], [0, 1]),             # not monotone / indptr[N] != E
    ([0, 2, 4], [0, 1, 1]),          # indptr[N] != E
    ([0, 2, 3], [0, 1, 2]),          # index out of range
    ([0, 2, 3], [0, -1, 1]),         # negative index
])
def test_bad_graphs_are_rejected(ip, ix):
    st, h = _create(ip, ix)
    assert st == capi.GA_ERR_BAD_GRAPH and not h.value


def test_bad_opts_are_rejected():
    # fields: light, hub threshold, hub chunk, build_csc, feature_slices, column hub
    # threshold, column hub chunk, row / column XCD split thresholds
    assert _create([0, 1], [0], capi.ga_plan_opts(1, 4, 8, 1, 0, 4, 8))[0] == capi.GA_OK
    assert _create([0, 1], [0], capi.ga_plan_opts(1, -1, -1, 1, 0, -1, -1))[0] == capi.GA_OK
    for bad in [(5, 4, 16, 1, 0, 8, 8),       # light > hub threshold
                (1, 4, 0, 1, 0, 4, 8),        # chunk 0
                (1, 4, -2, 1, 0, 4, 8),       # chunk below -1
                (-1, 4, 8, 1, 0, 4, 8),       # negative light
                (5, 8, 8, 1, 0, 4, 8),        # light > column hub threshold
                (1, 4, 8, 1, 0, 4, 0),        # column chunk 0
                (1, -4, 8, 1, 0, 4, 8),       # hub threshold below -1
                (1, 4, 8, 1, 3, 4, 8),        # feature slices not a power of two
                (1, 4, 8, 1, 16, 4, 8),       # too many feature slices
                (4, 8, 8, 1, 0, 8, 8, 2, 0),  # split threshold below light
                (4, 8, 8, 1, 0, 8, 8, 0, 3),  # column split threshold below light
                (4, 8, 8, 1, 0, 8, 8, -1, 0)]:  # negative split threshold
        assert _create([0, 1], [0], capi.ga_plan_opts(*bad))[0] == capi.GA_ERR_INVALID_ARG, bad
    assert capi.raw_status("graph_attn_plan_create", None, None, 0, 0, None, None) == \
        capi.GA_ERR_INVALID_ARG


def test_edge_count_limit():
    """E must stay at or below 2^31 - 2^16 (edge positions are 32-bit in the kernels, with
    room for a step past a row's end); larger counts are refused before any array is read."""
    ip, ix = np.array([0, 1], np.int32), np.array([0], np.int32)
    for e in (2 ** 31 - 2 ** 16 + 1, 2 ** 31, 2 ** 40):
        assert capi.raw_status("graph_attn_plan_create", ip.ctypes.data_as(POINTER(c_int32)),
                               ix.ctypes.data_as(POINTER(c_int32)), 1, e, None,
                               ctypes.byref(ctypes.c_void_p())) == capi.GA_ERR_INVALID_ARG, e


def test_empty_graph_plan():
    p = Plan(np.zeros(1, np.int32), np.zeros(0, np.int32))
    info = p.info()
    assert info["n_nodes"] == 0 and info["n_edges"] == 0 and info["uploaded"] == 0
    assert p.array("row_light").size == 0


def _hub_plan():
    rng = np.random.default_rng(0)
    ip, ix = gg.random_multigraph(64, 200, rng, hub_rows=(5,), hub_deg=300)
    return Plan(ip, ix, light_max_deg=4, hub_min_deg_exclusive=64, hub_chunk=32), ip, ix


FAKE = 1 << 20   # a 256-byte aligned address that is never dereferenced


def _fwd(p, score=capi.GA_SCORE_DOT, dtype=capi.GA_BF16, H=8, d=32, a=FAKE, b=FAKE, v=FAKE,
         out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30):
    return capi.raw_status("graph_attn_fwd", p.handle if p else None, score, dtype, H, d,
                           ctypes.c_float(0.1), ctypes.c_float(0.2), c_void_p(a), c_void_p(b),
                           c_void_p(v), c_void_p(out), c_void_p(lse), c_void_p(ws), wsb,
                           None)


def test_fwd_argument_checks_before_any_hip_call():
    p, _, _ = _hub_plan()
    assert p.info()["n_row_chunks"] > 0
    assert _fwd(None) == capi.GA_ERR_INVALID_ARG
    assert _fwd(p, score=7) == capi.GA_ERR_INVALID_ARG
    assert _fwd(p, dtype=9) == capi.GA_ERR_INVALID_ARG
    assert _fwd(p, H=0) == capi.GA_ERR_INVALID_ARG
    assert _fwd(p, d=12) == capi.GA_ERR_UNSUPPORTED        # 24-byte heads
    assert _fwd(p, H=16, d=64) == capi.GA_ERR_UNSUPPORTED  # 2 KB rows
    assert _fwd(p, dtype=capi.GA_F32, H=1, d=4) == capi.GA_ERR_UNSUPPORTED  # 16-byte heads
    assert _fwd(p, a=0) == capi.GA_ERR_INVALID_ARG
    assert _fwd(p, v=FAKE + 8) == capi.GA_ERR_INVALID_ARG   # misaligned
    assert _fwd(p, lse=0) == capi.GA_ERR_INVALID_ARG
    assert _fwd(p, score=capi.GA_SCORE_GAT, a=FAKE + 4, b=FAKE + 8) == capi.GA_ERR_NOT_READY
    assert _fwd(p, ws=0) == capi.GA_ERR_WORKSPACE
    need = p.fwd_workspace_bytes(8, 32)
    assert need > 0
    assert _fwd(p, wsb=need - 1) == capi.GA_ERR_WORKSPACE
    assert _fwd(p, wsb=need) == capi.GA_ERR_NOT_READY        # valid, but not uploaded


def _fwd_noalloc(p, score=capi.GA_SCORE_DOT, dtype=capi.GA_BF16, H=8, d=32, a=FAKE, b=FAKE,
                 v=FAKE, out=FAKE, lse=FAKE):
    return capi.raw_status("graph_attn_fwd_noalloc", p.handle if p else None, score, dtype, H,
                           d, ctypes.c_float(0.1), ctypes.c_float(0.2), c_void_p(a),
                           c_void_p(b), c_void_p(v), c_void_p(out), c_void_p(lse), None)


def test_fwd_noalloc_checks_and_scratch_limit_before_any_hip_call():
    p, _, _ = _hub_plan()
    assert _fwd_noalloc(None) == capi.GA_ERR_INVALID_ARG
    assert _fwd_noalloc(p, score=7) == capi.GA_ERR_INVALID_ARG
    assert _fwd_noalloc(p, d=12) == capi.GA_ERR_UNSUPPORTED
    assert _fwd_noalloc(p, a=0) == capi.GA_ERR_INVALID_ARG
    assert _fwd_noalloc(p, out=FAKE + 8) == capi.GA_ERR_INVALID_ARG
    assert _fwd_noalloc(p) == capi.GA_ERR_NOT_READY     # fits the scratch; not uploaded
    # a plan whose hub partials need more than the fixed scratch is refused as too large:
    # one hub row of one-edge chunks, each chunk's partial (m, l) and acc taking
    # (2 * 8 + 256) * 4 bytes at H = 8, d = 32
    n_chunks = capi.GA_FWD_NOALLOC_SCRATCH_BYTES // (256 * 4) + 1
    ip = np.array([0, n_chunks], np.int64)
    big = Plan(ip, np.zeros(n_chunks, np.int32), light_max_deg=0, hub_min_deg_exclusive=0,
               hub_chunk=1, build_csc=False)
    assert big.info()["n_row_chunks"] == n_chunks
    assert big.fwd_workspace_bytes(8, 32) > capi.GA_FWD_NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(big) == capi.GA_ERR_TOO_LARGE
    # the regular forward takes the same plan with a workspace of that size
    assert _fwd(big, wsb=big.fwd_workspace_bytes(8, 32)) == capi.GA_ERR_NOT_READY


def _bwd(p, score=capi.GA_SCORE_DOT, dtype=capi.GA_BF16, H=8, d=32, ptrs=None, ws=FAKE,
         wsb=1 << 30):
    ptrs = ptrs or [FAKE] * 8
    return capi.raw_status("graph_attn_bwd", p.handle, score, dtype, H, d, ctypes.c_float(0.1),
                           ctypes.c_float(0.2), *[c_void_p(x) for x in ptrs], c_void_p(ws), wsb,
                           None)


def test_bwd_argument_checks_before_any_hip_call():
    p, ip, ix = _hub_plan()
    assert _bwd(p, score=5) == capi.GA_ERR_INVALID_ARG
    assert _bwd(p, d=8, dtype=capi.GA_BF16) == capi.GA_ERR_UNSUPPORTED
    # GAT: s, t, ds, dt only need 4-byte alignment; v, dout, dv 16
    assert _bwd(p, score=capi.GA_SCORE_GAT, ptrs=[FAKE + 4, FAKE + 8, FAKE, FAKE, FAKE,
                                                  FAKE + 4, FAKE + 12, FAKE]) == capi.GA_ERR_NOT_READY
    assert _bwd(p, score=capi.GA_SCORE_GAT, ptrs=[FAKE, FAKE, FAKE + 4, FAKE, FAKE,
                                                  FAKE, FAKE, FAKE]) == capi.GA_ERR_INVALID_ARG
    assert _bwd(p, score=capi.GA_SCORE_DOT, ptrs=[FAKE + 4, FAKE, FAKE, FAKE, FAKE,
                                                  FAKE, FAKE, FAKE]) == capi.GA_ERR_INVALID_ARG
    for i in range(8):
        ptrs = [FAKE] * 8
        ptrs[i] = 0
        assert _bwd(p, ptrs=ptrs) == capi.GA_ERR_INVALID_ARG
    assert _bwd(p, ws=0) == capi.GA_ERR_WORKSPACE
    assert _bwd(p, wsb=p.bwd_workspace_bytes(8, 32) - 1) == capi.GA_ERR_WORKSPACE
    assert _bwd(p) == capi.GA_ERR_NOT_READY
    nocsc = Plan(ip, ix, build_csc=False)
    assert _bwd(nocsc) == capi.GA_ERR_NOT_READY
    assert nocsc.info()["has_csc"] == 0
    with pytest.raises(capi.GraphAttnError) as e:
        nocsc.array("rowidx")
    assert e.value.status == capi.GA_ERR_NOT_READY


def test_workspace_sizes_follow_the_declared_formulas():
    p, ip, ix = _hub_plan()
    info = p.info()
    al = lambda x: (x + 255) // 256 * 256
    H, d = 4, 64
    assert p.fwd_workspace_bytes(H, d) == al(info["n_row_chunks"] * H * 8) + \
        al(info["n_row_chunks"] * H * d * 4)
    assert p.bwd_workspace_bytes(H, d) == al(64 * H * 8) + \
        al(info["n_row_chunks"] * (2 * H * d + 8) * 4) + al(info["n_col_chunks"] * 2 * H * d * 4)
    assert p.bwd_workspace_bytes(8, 32) == al(64 * 8 * 8) + \
        al(info["n_row_chunks"] * (2 * 256 + 16) * 4) + al(info["n_col_chunks"] * 2 * 256 * 4)
    assert p.bwd_workspace_bytes(1, 64) == al(64 * 1 * 8) + \
        al(info["n_row_chunks"] * (2 * 64 + 4) * 4) + al(info["n_col_chunks"] * 2 * 64 * 4)
    # no hub rows -> no forward workspace
    q = Plan(*gg.csr_from_edges(4, [0, 1], [1, 2]))
    assert q.fwd_workspace_bytes(8, 32) == 0


def test_plan_arrays_and_upload_checks():
    p, ip, ix = _hub_plan()
    names = [capi.graph_attn_plan_array_name(i).decode()
             for i in range(capi.graph_attn_plan_array_count())]
    assert names[:2] == ["indptr", "indices"] and "rowidx" in names
    assert capi.graph_attn_plan_array_name(999) is None
    assert np.array_equal(p.array("indptr"), ip) and np.array_equal(p.array("indices"), ix)
    with pytest.raises(capi.GraphAttnError):
        p.array("nope")
    # misaligned or too-small device buffer: rejected before touching HIP
    assert capi.raw_status("graph_attn_plan_upload", p.handle, c_void_p(FAKE + 16),
                           1 << 30, None) == capi.GA_ERR_INVALID_ARG
    assert capi.raw_status("graph_attn_plan_upload", p.handle, c_void_p(FAKE),
                           16, None) == capi.GA_ERR_INVALID_ARG


def test_timers_and_copy_probe_host_paths():
    assert capi.raw_status("graph_attn_timer_enable", 1) == 0
    assert capi.graph_attn_timer_count() == 0
    assert capi.raw_status("graph_attn_timer_read", 0, None, None, None) == \
        capi.GA_ERR_INVALID_ARG
    assert capi.raw_status("graph_attn_timer_reset") == 0
    assert capi.raw_status("graph_attn_timer_enable", 0) == 0
    assert capi.raw_status("graph_attn_copy_probe", c_void_p(FAKE), c_void_p(FAKE), 17,
                           None) == capi.GA_ERR_INVALID_ARG
    assert capi.raw_status("graph_attn_copy_probe", c_void_p(FAKE + 8), c_void_p(FAKE), 32,
                           None) == capi.GA_ERR_INVALID_ARG


def test_gather_probe_argument_checks():
    p, ip, ix = _hub_plan()
    call = lambda plan, H=8, d=32, a=FAKE, b=0, k=FAKE, v=FAKE, sink=FAKE: capi.raw_status(
        "graph_attn_gather_probe", plan.handle if plan else None, capi.GA_BF16, H, d,
        c_void_p(a), c_void_p(b), c_void_p(k), c_void_p(v), c_void_p(sink), None)
    assert call(None) == capi.GA_ERR_INVALID_ARG
    assert call(p, d=12) == capi.GA_ERR_UNSUPPORTED
    assert call(p, k=0) == capi.GA_ERR_INVALID_ARG
    assert call(p, a=FAKE + 8) == capi.GA_ERR_INVALID_ARG
    assert call(p, sink=FAKE + 4) == capi.GA_ERR_INVALID_ARG
    assert call(p) == capi.GA_ERR_NOT_READY
    assert call(p, a=0, v=0) == capi.GA_ERR_NOT_READY          # optional operands
    cols = lambda plan, k=0, v=0, q=FAKE, dout=FAKE, rec=FAKE, sink=FAKE: capi.raw_status(
        "graph_attn_gather_probe_cols", plan.handle if plan else None, capi.GA_BF16, 8, 32,
        c_void_p(k), c_void_p(v), c_void_p(q), c_void_p(dout), c_void_p(rec), c_void_p(sink),
        None)
    assert cols(None) == capi.GA_ERR_INVALID_ARG
    assert cols(p, dout=0) == capi.GA_ERR_INVALID_ARG
    assert cols(p, rec=FAKE + 4) == capi.GA_ERR_INVALID_ARG
    assert cols(p, q=FAKE + 8) == capi.GA_ERR_INVALID_ARG
    assert cols(p) == capi.GA_ERR_NOT_READY
    assert cols(Plan(ip, ix, build_csc=False)) == capi.GA_ERR_NOT_READY
    rnd = lambda rb=512, t=FAKE, rows=100, n=10, sink=FAKE: capi.raw_status(
        "graph_attn_gather_probe_random", rb, c_void_p(t), rows, n, 7, c_void_p(sink), None)
    assert rnd(rb=48) == capi.GA_ERR_UNSUPPORTED
    assert rnd(rows=0) == capi.GA_ERR_INVALID_ARG
    assert rnd(rows=1 << 32) == capi.GA_ERR_INVALID_ARG
    assert rnd(n=-1) == capi.GA_ERR_INVALID_ARG
    assert rnd(t=FAKE + 8) == capi.GA_ERR_INVALID_ARG
    assert rnd(n=0) == capi.GA_OK                               # nothing to launch


def test_fwd_gatv2_argument_checks():
    p, _, _ = _hub_plan()
    call = lambda H=8, d=32, xd=FAKE, xs=FAKE, attn=FAKE, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30: \
        capi.raw_status("graph_attn_fwd_gatv2", p.handle, capi.GA_BF16, H, d, ctypes.c_float(1.0),
                        ctypes.c_float(0.2), c_void_p(xd), c_void_p(xs), c_void_p(attn),
                        c_void_p(out), c_void_p(lse), c_void_p(ws), wsb, None)
    assert call(d=12) == capi.GA_ERR_UNSUPPORTED
    assert call(attn=0) == capi.GA_ERR_INVALID_ARG
    assert call(attn=FAKE + 4) == capi.GA_ERR_INVALID_ARG
    assert call(xs=FAKE + 8) == capi.GA_ERR_INVALID_ARG
    assert call(ws=0) == capi.GA_ERR_WORKSPACE
    assert call() == capi.GA_ERR_NOT_READY


def test_bwd_gatv2_argument_checks():
    p, ip, ix = _hub_plan()
    need = c_size_t()
    capi.graph_attn_bwd_gatv2_workspace_bytes(p.handle, capi.GA_BF16, 8, 32, byref(need))
    info = p.info()
    al = lambda x: (x + 255) // 256 * 256
    slots = 0
    for side in ("row", "col"):     # one slot per 16 work items, plus one per hub
        items = info[f"n_{side}_chunks"] + info[f"n_{side}_medium"] + -(-info[f"n_{side}_light"] // 2)
        slots += -(-items // 16) + info[f"n_{side}_hub"]
    r64 = -(-slots // 32) + -(-slots // 1024)
    assert need.value == al(64 * 8 * 8) + al(info["n_row_chunks"] * (2 * 256 + 16) * 4) + \
        al(info["n_col_chunks"] * 2 * 256 * 4) + al(slots * 256 * 4) + al(r64 * 256 * 8)

    def call(ptrs=None, attn=FAKE, dattn=FAKE, ws=FAKE, wsb=1 << 30, plan=p):
        ptrs = ptrs or [FAKE] * 6
        return capi.raw_status("graph_attn_bwd_gatv2", plan.handle, capi.GA_BF16, 8, 32,
                               ctypes.c_float(1.0), ctypes.c_float(0.2), c_void_p(ptrs[0]),
                               c_void_p(ptrs[1]), c_void_p(attn), c_void_p(ptrs[2]),
                               c_void_p(ptrs[3]), c_void_p(ptrs[4]), c_void_p(ptrs[5]),
                               c_void_p(dattn), c_void_p(ws), wsb, None)
    assert call(attn=0) == capi.GA_ERR_INVALID_ARG
    assert call(dattn=FAKE + 4) == capi.GA_ERR_INVALID_ARG
    for i in range(6):
        ptrs = [FAKE] * 6
        ptrs[i] = 0
        assert call(ptrs) == capi.GA_ERR_INVALID_ARG
    assert call(wsb=need.value - 1) == capi.GA_ERR_WORKSPACE
    assert call(wsb=need.value) == capi.GA_ERR_NOT_READY
    assert call(plan=Plan(ip, ix, build_csc=False)) == capi.GA_ERR_NOT_READY


def test_default_opts():
    o = default_opts()
    assert o["build_csc"] == 1
    # -1 = chosen from the graph's size
    assert (o["light_max_deg"], o["hub_min_deg_exclusive"], o["hub_chunk"]) == (16, -1, -1)
    assert (o["col_hub_min_deg_exclusive"], o["col_hub_chunk"]) == (-1, -1)
    assert o["feature_slices"] == 0
    # the binding: explicit row thresholds also set the columns unless given
    rng = np.random.default_rng(3)
    ip, ix = gg.random_multigraph(64, 200, rng, hub_rows=(5,), hub_deg=300)
    i = Plan(ip, ix, hub_min_deg_exclusive=64, hub_chunk=32).info()
    assert (i["col_hub_min_deg_exclusive"], i["col_hub_chunk"]) == (64, 32)
    i = Plan(ip, ix, hub_min_deg_exclusive=64, col_hub_chunk=7).info()
    assert (i["hub_chunk"], i["col_hub_min_deg_exclusive"], i["col_hub_chunk"]) == (256, 64, 7)
    i = Plan(ip, ix).info()        # 264 edges: the smallest automatic values
    assert (i["hub_min_deg_exclusive"], i["hub_chunk"], i["col_hub_min_deg_exclusive"],
            i["col_hub_chunk"]) == (256, 256, 256, 256)


def _auto(e, light=16):
    """The documented automatic thresholds, restated: the power of two nearest E/8192 in
    [256, 8192] (nearest on a log scale), chunk max(256, t/4), columns min(1024, t) and
    min(512, chunk)."""
    import math
    share = e / 8192
    t = 256
    while t < 8192 and t * math.sqrt(2) < share:
        t *= 2
    t = max(t, light)
    c = max(256, t // 4)
    return t, c, max(min(1024, t), light), min(512, c)


@pytest.mark.parametrize("e", [0, 100, 2_100_000, 2_966_000, 2_967_000, 16_000_000,
                               51_000_000, 65_000_000, 500_000_000])
def test_automatic_thresholds(e):
    # a star-free CSR with e edges spread over rows; only the edge count matters
    n = 1000
    ip = (np.arange(n + 1, dtype=np.int64) * e // n).astype(np.int32)
    ix = np.zeros(e, np.int32)
    st, h = _create(ip, ix, None) if e <= 2_000_000 else (None, None)
    if st is None:                     # build the big ones through the binding (same call)
        p = Plan(ip, ix, build_csc=False)
        i = p.info()
    else:
        assert st == capi.GA_OK
        info = capi.ga_plan_info()
        capi.graph_attn_plan_get_info(h, byref(info))
        i = info.as_dict()
        capi.graph_attn_plan_destroy(h)
    got = (i["hub_min_deg_exclusive"], i["hub_chunk"], i["col_hub_min_deg_exclusive"],
           i["col_hub_chunk"])
    assert got == _auto(e), (e, got)
    assert _auto(51_000_000)[:2] == (8192, 2048) and _auto(2_100_000)[:2] == (256, 256)


def _rfwd(p, op=capi.GA_REDUCE_MAX, dtype=capi.GA_BF16, F=256, ptrs=None, slot=FAKE, ws=FAKE,
          wsb=1 << 30):
    ptrs = ptrs or [FAKE] * 3
    return capi.raw_status("graph_attn_reduce_fwd", p.handle if p else None, op, dtype, F,
                           *[c_void_p(x) for x in ptrs], c_void_p(slot), c_void_p(ws), wsb,
                           None)


def _rbwd(p, dtype=capi.GA_BF16, F=256, ptrs=None, ws=FAKE, wsb=1 << 30):
    ptrs = ptrs or [FAKE] * 4           # arg, slot, dout, dx
    return capi.raw_status("graph_attn_reduce_bwd", p.handle if p else None, dtype, F,
                           *[c_void_p(x) for x in ptrs], c_void_p(ws), wsb, None)


def _rws(p, fn, F):
    b = c_size_t()
    assert capi.raw_status(fn, p.handle, F, byref(b)) == capi.GA_OK
    return b.value


def test_reduce_argument_checks_before_any_hip_call():
    rng = np.random.default_rng(1)
    src = np.concatenate([rng.integers(0, 64, 200), np.full(300, 9), rng.integers(0, 64, 300)])
    dst = np.concatenate([rng.integers(0, 64, 200), rng.integers(0, 64, 300), np.full(300, 5)])
    ip, ix = gg.csr_from_edges(64, src, dst)     # node 5: hub row, node 9: hub column
    p = Plan(ip, ix, light_max_deg=4, hub_min_deg_exclusive=64, hub_chunk=32)
    info = p.info()
    al = lambda x: (x + 255) // 256 * 256
    assert info["n_row_chunks"] > 0 and info["n_col_chunks"] > 0
    # declared workspace formulas
    for F in (16, 64, 256, 512):
        assert _rws(p, "graph_attn_reduce_fwd_workspace_bytes", F) == \
            3 * al(info["n_row_chunks"] * F * 4)
        assert _rws(p, "graph_attn_reduce_bwd_workspace_bytes", F) == \
            al(info["n_col_chunks"] * F * 4)
    nfw = _rws(p, "graph_attn_reduce_fwd_workspace_bytes", 256)
    nbw = _rws(p, "graph_attn_reduce_bwd_workspace_bytes", 256)
    assert _rfwd(None) == capi.GA_ERR_INVALID_ARG
    assert _rfwd(p, op=2) == capi.GA_ERR_INVALID_ARG
    assert _rfwd(p, dtype=5) == capi.GA_ERR_INVALID_ARG
    assert _rfwd(p, F=0) == capi.GA_ERR_INVALID_ARG
    assert _rfwd(p, F=12) == capi.GA_ERR_UNSUPPORTED               # 24-byte rows
    assert _rfwd(p, F=1024) == capi.GA_ERR_UNSUPPORTED             # 2 KB rows
    assert _rfwd(p, F=24) == capi.GA_ERR_UNSUPPORTED               # 48 B: 3 lanes
    assert _rfwd(p, dtype=capi.GA_F32, F=8) == capi.GA_ERR_UNSUPPORTED  # 32 B: 2 lanes
    for i in range(3):
        ptrs = [FAKE] * 3
        ptrs[i] = 0
        assert _rfwd(p, ptrs=ptrs) == capi.GA_ERR_INVALID_ARG
        ptrs[i] = FAKE + 8
        assert _rfwd(p, ptrs=ptrs) == capi.GA_ERR_INVALID_ARG
    assert _rfwd(p, slot=0) == capi.GA_ERR_NOT_READY               # slot is optional
    assert _rfwd(p, slot=FAKE + 8) == capi.GA_ERR_INVALID_ARG       # but aligned if given
    assert _rfwd(p, ws=0) == capi.GA_ERR_WORKSPACE
    assert _rfwd(p, wsb=nfw - 1) == capi.GA_ERR_WORKSPACE
    assert _rfwd(p, wsb=nfw) == capi.GA_ERR_NOT_READY               # valid, not uploaded
    assert _rfwd(p, op=capi.GA_REDUCE_MIN, dtype=capi.GA_F32, F=64) == capi.GA_ERR_NOT_READY
    # backward
    assert _rbwd(None) == capi.GA_ERR_INVALID_ARG
    assert _rbwd(p, F=12) == capi.GA_ERR_UNSUPPORTED
    assert _rbwd(p, ptrs=[0, FAKE, FAKE, FAKE]) == capi.GA_ERR_NOT_READY   # slot replaces arg
    assert _rbwd(p, ptrs=[FAKE, 0, FAKE, FAKE]) == capi.GA_ERR_NOT_READY   # arg without slot
    assert _rbwd(p, ptrs=[0, 0, FAKE, FAKE]) == capi.GA_ERR_INVALID_ARG    # neither
    assert _rbwd(p, ptrs=[FAKE, FAKE + 4, FAKE, FAKE]) == capi.GA_ERR_INVALID_ARG
    for i in (2, 3):
        ptrs = [FAKE] * 4
        ptrs[i] = 0
        assert _rbwd(p, ptrs=ptrs) == capi.GA_ERR_INVALID_ARG
    assert _rbwd(p, wsb=nbw - 1) == capi.GA_ERR_WORKSPACE
    assert _rbwd(p, wsb=nbw) == capi.GA_ERR_NOT_READY
    assert _rbwd(Plan(ip, ix, build_csc=False)) == capi.GA_ERR_NOT_READY
    # a graph without hub rows needs no workspace, and NULL is accepted for it
    q = Plan(*gg.csr_from_edges(4, [0, 1], [1, 2]))
    assert _rws(q, "graph_attn_reduce_fwd_workspace_bytes", 256) == 0
    assert _rws(q, "graph_attn_reduce_bwd_workspace_bytes", 256) == 0
    assert _rfwd(q, ws=0, wsb=0) == capi.GA_ERR_NOT_READY
    assert _rbwd(q, ws=0, wsb=0) == capi.GA_ERR_NOT_READY
    # slot width: 2 bytes unless some row has more than 65535 edges (positions up to 65534,
    # so none equals the all-ones slot of an element without a winner)
    b = c_size_t()
    capi.graph_attn_reduce_slot_bytes(p.handle, byref(b))
    assert b.value == 2
    big = Plan(*gg.csr_from_edges(3, np.zeros(65536, np.int64), np.full(65536, 1)))
    capi.graph_attn_reduce_slot_bytes(big.handle, byref(b))
    assert b.value == 4
    ok = Plan(*gg.csr_from_edges(3, np.zeros(65535, np.int64), np.full(65535, 1)))
    capi.graph_attn_reduce_slot_bytes(ok.handle, byref(b))
    assert b.value == 2


def test_missing_library_fails_loudly():
    """Without the built HIP library the package raises on first use: there is no CPU
    fallback (a fresh process pointed at a library path that does not exist)."""
    import subprocess
    import sys
    code = ("import numpy as np, sparse_graph_attention_02_amd as ga\n"
            "try:\n"
            "    ga.Plan(np.array([0, 1], np.int32), np.array([0], np.int32))\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n")
    env = dict(os.environ, GRAPH_ATTN_LIB="/nonexistent/libgraph_attn.so")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "missing" in r.stdout, r.stdout


def test_reduce_accepts_xcd_split_plans():
    """Split plans pass the reduction's argument checks (an upload is what is missing)."""
    ip, ix = gg.make_graph(gg.WORKLOADS["chunglu100k_gat_f32"], n=5_000)
    for xs, cxs in [(32, 0), (0, 32), (32, 32)]:
        p = Plan(ip, ix, xcd_split_min_deg_exclusive=xs, col_xcd_split_min_deg_exclusive=cxs)
        assert _rfwd(p) == capi.GA_ERR_NOT_READY
        assert _rbwd(p) == capi.GA_ERR_NOT_READY


def test_xcd_split_defaults_and_info():
    """The split is off by default; a split plan reports its thresholds and schedule sizes
    (multiples of 8 XCDs x 4 wavefronts), and the workspace formulas follow its chunks."""
    from sparse_graph_attention_02_amd import default_opts
    d = default_opts()
    assert d["xcd_split_min_deg_exclusive"] == 0 and d["col_xcd_split_min_deg_exclusive"] == 0
    ip, ix = gg.make_graph(gg.WORKLOADS["chunglu100k_gat_f32"], n=5_000)
    plain = Plan(ip, ix).info()
    assert plain["n_row_sched"] == 0 and plain["n_col_sched"] == 0
    p = Plan(ip, ix, xcd_split_min_deg_exclusive=32, col_xcd_split_min_deg_exclusive=64)
    info = p.info()
    assert info["xcd_split_min_deg_exclusive"] == 32
    assert info["col_xcd_split_min_deg_exclusive"] == 64
    assert info["n_row_sched"] > 0 and info["n_row_sched"] % 32 == 0
    assert info["n_col_sched"] > 0 and info["n_col_sched"] % 32 == 0
    assert p.array("row_sched").size == info["n_row_sched"]
    deg = np.diff(ip)
    assert info["n_row_hub"] == int(np.sum(deg > 32))
    al = lambda x: (x + 255) // 256 * 256
    nc = info["n_row_chunks"]
    assert p.fwd_workspace_bytes(8, 32) == al(nc * 8 * 2 * 4) + al(nc * 256 * 4)


@pytest.mark.parametrize("tx,c", [(16, 4), (32, 16), (256, 2048), (64, 64)])
def test_split_chunk_count_bound(tx, c):
    """Upper bound on a split plan's chunks, hence on the hub workspaces: a split row of d
    edges (d > T_X) gives at most d / C + 8 chunks (eight residue groups, each cut into
    C-edge chunks), an unsplit hub row at most d / C + 1, and at most E / (T_X + 1) rows
    are split, so chunks <= E / C + 8 E / (T_X + 1) + E / (T_H + 1). Checked on a power-law
    graph and on the adversarial one where every row has T_X + 1 edges."""
    rng = np.random.default_rng(tx)
    graphs = [gg.make_graph(gg.WORKLOADS["chunglu1m_dot_bf16"], n=4000)]
    n = 600
    src = rng.integers(0, n, n * (tx + 1))
    dst = np.repeat(np.arange(n), tx + 1)
    graphs.append(gg.csr_from_edges(n, src, dst))
    for ip, ix in graphs:
        E = ix.size
        p = Plan(ip, ix, light_max_deg=min(16, tx), hub_min_deg_exclusive=max(tx, 16) * 4,
                 hub_chunk=c, xcd_split_min_deg_exclusive=tx, col_xcd_split_min_deg_exclusive=tx,
                 col_hub_chunk=c)
        info = p.info()
        for side, th in (("row", info["hub_min_deg_exclusive"]),
                         ("col", info["col_hub_min_deg_exclusive"])):
            bound = E / c + 8 * E / (tx + 1) + E / (th + 1)
            assert info[f"n_{side}_chunks"] <= bound, (side, info[f"n_{side}_chunks"], bound)
