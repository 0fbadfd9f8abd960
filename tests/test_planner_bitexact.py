"""The library's C++ planner (through the C ABI, host only) against the numpy reference
planner of the oracle: every plan array must be identical."""
import numpy as np
import pytest

import graphgen as gg
from oracle import planner as P
from sparse_graph_attention_02_amd import Plan, capi

NAMES = None


def _names():
    return [capi.graph_attn_plan_array_name(i).decode()
            for i in range(capi.graph_attn_plan_array_count())]


def _graphs():
    rng = np.random.default_rng(1)
    yield "star", gg.csr_from_edges(300, np.arange(300), np.zeros(300, np.int64))
    yield "multigraph_hubs", gg.random_multigraph(500, 4000, rng, hub_rows=(0, 17, 499),
                                                  hub_deg=1500)
    yield "empty_rows", gg.csr_from_edges(40, rng.integers(0, 40, 50), rng.integers(0, 5, 50))
    yield "no_edges", (np.zeros(9, np.int32), np.zeros(0, np.int32))
    yield "no_nodes", (np.zeros(1, np.int32), np.zeros(0, np.int32))
    yield "chunglu30k", gg.make_graph(gg.WORKLOADS["chunglu100k_gat_f32"], n=30_000)
    yield "rmat2^14", gg.make_graph(gg.WORKLOADS["rmat21_dot_bf16"], n=1 << 14)
    # one row holding nearly every edge: most of the transpose's row blocks are empty
    yield "giant_row", gg.csr_from_edges(
        1000, np.r_[rng.integers(0, 1000, 90_000), rng.integers(0, 1000, 500)],
        np.r_[np.full(90_000, 5), rng.integers(0, 1000, 500)])


THRESH = [(16, 1024, 512), (0, 0, 1), (2, 3, 2), (31, 32, 33), (8, 64, 64)]


@pytest.mark.parametrize("name,g", list(_graphs()), ids=lambda x: x if isinstance(x, str) else "")
@pytest.mark.parametrize("tl,th,c", THRESH)
def test_cpp_planner_equals_reference(name, g, tl, th, c):
    ip, ix = g
    ref = P.plan(ip, ix, tl, th, c, build_csc=True)
    p = Plan(ip, ix, light_max_deg=tl, hub_min_deg_exclusive=th, hub_chunk=c)
    for nm in _names():
        got = p.array(nm)
        want = {"indptr": ip, "indices": ix}.get(nm, ref.get(nm))
        assert got.dtype == np.int32
        assert np.array_equal(got, np.asarray(want, np.int32)), nm
    info = p.info()
    n = ip.size - 1
    assert info["n_row_hub"] == ref["row_hub"].size
    ixs = np.asarray(ix, np.int64)
    same_row = np.repeat(np.arange(n), np.diff(ip))
    srt = not np.any((np.diff(ixs) < 0) & (same_row[1:] == same_row[:-1])) if ixs.size else True
    assert info["rows_sorted"] == int(srt)
    assert info["max_in_degree"] == (int(np.diff(ip).max()) if n else 0)


def test_threshold_edges_and_chunk_multiples():
    """Rows with degree exactly at, below and above the thresholds; hub rows whose degree
    is a multiple of the chunk and one more / one less."""
    tl, th, c = 4, 16, 8
    degs = [0, 1, tl - 1, tl, tl + 1, th - 1, th, th + 1, 2 * c + 16, 3 * c, 3 * c - 1,
            3 * c + 1, 5 * c]
    n = len(degs)
    rng = np.random.default_rng(2)
    dst = np.repeat(np.arange(n), degs)
    src = rng.integers(0, n, dst.size)
    ip, ix = gg.csr_from_edges(n, src, dst)
    ref = P.plan(ip, ix, tl, th, c)
    p = Plan(ip, ix, light_max_deg=tl, hub_min_deg_exclusive=th, hub_chunk=c)
    for nm in _names():
        want = {"indptr": ip, "indices": ix}.get(nm, ref.get(nm))
        assert np.array_equal(p.array(nm), want), nm
    assert sorted(p.array("row_light").tolist()) == [0, 1, 2, 3]
    assert sorted(p.array("row_medium").tolist()) == [4, 5, 6]
    chunks = np.diff(p.array("row_hub_chunk_ptr"))
    hub = p.array("row_hub")
    expect = {i: -(-degs[i] // c) for i in hub}
    assert [expect[i] for i in hub] == chunks.tolist()


def test_rows_sorted_flag():
    ip = np.array([0, 2, 4, 5])
    assert Plan(ip, np.array([0, 1, 2, 2, 1])).info()["rows_sorted"] == 1
    assert Plan(ip, np.array([1, 0, 2, 2, 1])).info()["rows_sorted"] == 0
    assert Plan(ip, np.array([0, 1, 2, 0, 1])).info()["rows_sorted"] == 0
    assert Plan(np.array([0, 2, 3]), np.array([1, 1, 0])).info()["rows_sorted"] == 1


@pytest.mark.parametrize("name,g", list(_graphs()), ids=lambda x: x if isinstance(x, str) else "")
@pytest.mark.parametrize("tl,th,c,cth,cc", [(16, 8192, 2048, 1024, 512), (4, 64, 16, 8, 3),
                                            (2, 3, 2, 100, 50)])
def test_cpp_planner_column_thresholds(name, g, tl, th, c, cth, cc):
    """Rows and columns binned with their own hub threshold and chunk."""
    ip, ix = g
    ref = P.plan(ip, ix, tl, th, c, build_csc=True, col_hub_min_deg_exclusive=cth,
                 col_hub_chunk=cc)
    p = Plan(ip, ix, light_max_deg=tl, hub_min_deg_exclusive=th, hub_chunk=c,
             col_hub_min_deg_exclusive=cth, col_hub_chunk=cc)
    for nm in _names():
        want = {"indptr": ip, "indices": ix}.get(nm, ref.get(nm))
        assert np.array_equal(p.array(nm), np.asarray(want, np.int32)), nm


@pytest.mark.parametrize("name,g", list(_graphs()), ids=lambda x: x if isinstance(x, str) else "")
@pytest.mark.parametrize("tl,th,c,xs,cxs", [(16, 8192, 2048, 64, 64), (4, 64, 16, 8, 100),
                                            (2, 3, 2, 2, 0), (0, 1000, 7, 0, 5),
                                            (8, 16, 1, 300, 40)])
def test_cpp_planner_xcd_split(name, g, tl, th, c, xs, cxs):
    """Rows / columns regrouped by neighbour id mod 8, chunked per group and scheduled to
    XCD slots: every array identical to the reference planner's."""
    ip, ix = g
    ref = P.plan(ip, ix, tl, th, c, build_csc=True, xcd_split=xs, col_xcd_split=cxs)
    p = Plan(ip, ix, light_max_deg=tl, hub_min_deg_exclusive=th, hub_chunk=c,
             xcd_split_min_deg_exclusive=xs, col_xcd_split_min_deg_exclusive=cxs)
    for nm in _names():
        assert np.array_equal(p.array(nm), np.asarray(ref[nm], np.int32)), nm
    info = p.info()
    assert info["n_row_sched"] == ref["row_sched"].size
    assert info["n_col_sched"] == ref["col_sched"].size


def test_xcd_split_invariants():
    """What the split must keep, checked on the library's plan directly: each row's
    neighbour multiset; each split chunk draws from one partition; the schedule runs every
    chunk exactly once and puts partition p's chunks in workgroups w = p (mod 8); the
    transpose is the transpose of the regrouped CSR."""
    ip, ix = gg.make_graph(gg.WORKLOADS["chunglu100k_gat_f32"], n=30_000)
    xs = 40
    p = Plan(ip, ix, light_max_deg=8, hub_min_deg_exclusive=512, hub_chunk=128,
             xcd_split_min_deg_exclusive=xs)
    pix = p.array("indices")
    deg = np.diff(ip)
    for i in range(ip.size - 1):
        a, b = ip[i], ip[i + 1]
        assert np.array_equal(np.sort(pix[a:b]), np.sort(ix[a:b]))
        if deg[i] <= xs:
            assert np.array_equal(pix[a:b], ix[a:b])
    cr, cb, ce = p.array("row_chunk_row"), p.array("row_chunk_begin"), p.array("row_chunk_end")
    sched = p.array("row_sched")
    assert sched.size % 32 == 0 and sched.size > 0
    run = sched[sched >= 0]
    assert np.array_equal(np.sort(run), np.arange(cr.size))
    for slot, c in enumerate(sched):
        if c < 0 or deg[cr[c]] <= xs:
            continue
        parts = np.unique(pix[cb[c]:ce[c]] % 8)
        assert parts.size == 1 and parts[0] == (slot // 4) % 8
    colptr, rowidx = P.transpose(ip, pix)
    assert np.array_equal(p.array("colptr"), colptr)
    # columns follow the row split threshold; their groups hold destinations of one class
    cpix = p.array("rowidx")
    for j in np.flatnonzero(np.diff(colptr) > xs)[:50]:
        a, b = colptr[j], colptr[j + 1]
        assert np.array_equal(np.sort(cpix[a:b]), np.sort(rowidx[a:b]))
        assert np.all(np.diff(cpix[a:b] % 8) >= 0)
