"""Pins of the reference planner: scipy's CSR->CSC conversion, partition invariants,
chunk tiling and CSR validation."""
import numpy as np
import pytest
import scipy.sparse as sp

import graphgen as gg
from oracle import planner as P


def _graphs():
    rng = np.random.default_rng(0)
    yield "multigraph", gg.random_multigraph(200, 3000, rng, hub_rows=(3, 77), hub_deg=700)
    yield "empty_rows", gg.csr_from_edges(50, rng.integers(0, 50, 80), rng.integers(0, 10, 80))
    yield "no_edges", (np.zeros(6, np.int32), np.zeros(0, np.int32))
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    yield "chunglu20k", gg.make_graph(w, n=20_000)


@pytest.mark.parametrize("name,g", list(_graphs()), ids=lambda x: x if isinstance(x, str) else "")
def test_transpose_matches_scipy(name, g):
    ip, ix = g
    n = ip.size - 1
    colptr, rowidx = P.transpose(ip, ix)
    eid = np.arange(ix.size, dtype=np.int64)
    m = sp.csr_matrix((eid, ix, ip), shape=(n, n)).tocsc()
    assert np.array_equal(colptr, m.indptr)
    assert np.array_equal(rowidx, m.indices)
    # each CSC slot names the CSR edge it came from: same (row, col) and stable order
    edge_row = np.repeat(np.arange(n), np.diff(ip))
    assert np.array_equal(edge_row[m.data], rowidx)
    # stable: within a column, CSR edge ids (hence destinations) ascend
    col_of_slot = np.repeat(np.arange(n), np.diff(colptr))
    same_col = col_of_slot[1:] == col_of_slot[:-1]
    assert np.all(np.diff(m.data)[same_col] > 0)
    assert np.all(np.diff(rowidx)[same_col] >= 0)
    # and its position within the CSR row it came from
    rel = P.transpose_positions(ip, ix)
    assert np.array_equal(rel, m.data - np.asarray(ip, np.int64)[rowidx])
    assert np.array_equal(np.asarray(ix)[np.asarray(ip, np.int64)[rowidx] + rel],
                          col_of_slot)


@pytest.mark.parametrize("name,g", list(_graphs()), ids=lambda x: x if isinstance(x, str) else "")
@pytest.mark.parametrize("tl,th,c", [(16, 256, 128), (1, 1, 1), (0, 100, 37), (32, 1024, 1024)])
def test_bins_partition_and_chunks_tile(name, g, tl, th, c):
    ip, ix = g
    n = ip.size - 1
    plan = P.plan(ip, ix, tl, th, c)
    deg = np.diff(ip.astype(np.int64))
    allrows = np.concatenate([plan["row_light"], plan["row_medium"], plan["row_hub"]])
    assert np.array_equal(np.sort(allrows), np.arange(n))
    assert np.all(deg[plan["row_light"]] <= tl)
    assert np.all((deg[plan["row_medium"]] > tl) & (deg[plan["row_medium"]] <= th))
    assert np.all(deg[plan["row_hub"]] > th)
    for b in ("row_light", "row_medium", "row_hub"):
        r = plan[b].astype(np.int64)
        key = -deg[r] * (n + 1) + r          # degree descending, then id ascending
        assert np.all(np.diff(key) > 0)
    ptr = plan["row_hub_chunk_ptr"]
    assert ptr.size == plan["row_hub"].size + 1 and ptr[0] == 0
    for h, i in enumerate(plan["row_hub"]):
        b, e = plan["row_chunk_begin"][ptr[h]:ptr[h + 1]], plan["row_chunk_end"][ptr[h]:ptr[h + 1]]
        assert np.all(plan["row_chunk_row"][ptr[h]:ptr[h + 1]] == i)
        assert b[0] == ip[i] and e[-1] == ip[i + 1]
        assert np.array_equal(b[1:], e[:-1]) and np.all(e - b <= c) and np.all(e > b)
    odeg = np.bincount(ix, minlength=n)
    assert np.array_equal(np.sort(np.concatenate(
        [plan["col_light"], plan["col_medium"], plan["col_hub"]])), np.arange(n))
    assert np.all(odeg[plan["col_hub"]] > th)
    assert plan["col_chunk_end"].sum() - plan["col_chunk_begin"].sum() == odeg[plan["col_hub"]].sum()


def test_validate_csr():
    ip = np.array([0, 2, 3], np.int32)
    ix = np.array([1, 0, 1], np.int32)
    assert P.validate_csr(ip, ix)
    assert not P.validate_csr(np.array([1, 2, 3]), ix)           # indptr[0] != 0
    assert not P.validate_csr(np.array([0, 3, 2]), ix[:2])       # not monotone
    assert not P.validate_csr(np.array([0, 2, 4]), ix)           # indptr[N] != E
    assert not P.validate_csr(ip, np.array([1, 0, 2], np.int32))  # index out of range
    assert not P.validate_csr(ip, np.array([1, -1, 0], np.int32))


def test_xcd_split_worked_example():
    """The reference planner's XCD split against a hand-worked example
    (tests/golden/xcd_split_example.json)."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "xcd_split_example.json")))
    o = g["options"]
    got = P.plan(g["indptr"], g["indices"], o["light_max_deg"], o["hub_min_deg_exclusive"],
                 o["hub_chunk"], build_csc=False, xcd_split=o["xcd_split"])
    for name, want in g["expected"].items():
        assert np.array_equal(got[name], np.asarray(want, np.int32)), name


@pytest.mark.parametrize("name,g", list(_graphs()), ids=lambda x: x if isinstance(x, str) else "")
@pytest.mark.parametrize("xs,cxs,chunk", [(8, 8, 5), (40, 16, 1000), (2, 0, 1)])
def test_xcd_split_invariants_of_the_reference_planner(name, g, xs, cxs, chunk):
    """What the split must keep, on the reference planner itself: each row's and column's
    multiset; rows / columns above the threshold are hubs grouped by residue mod 8 (stable
    within a group) and every chunk lies inside one group; unsplit rows keep their order;
    the schedule runs every chunk once, partition p's chunks in workgroups = p (mod 8),
    each partition's chunks longest first; the transpose is that of the regrouped CSR."""
    ip, ix = g
    ip64, ix64 = np.asarray(ip, np.int64), np.asarray(ix, np.int64)
    n = ip64.size - 1
    out = P.plan(ip, ix, 0, 10**9, chunk, build_csc=True, xcd_split=xs, col_xcd_split=cxs)
    for side, ptr, orig, key, thr in (("row", ip64, ix64, out["indices"], xs),
                                      ("col", out["colptr"].astype(np.int64),
                                       P.transpose(ip, out["indices"])[1], out["rowidx"], cxs)):
        deg = np.diff(ptr)
        cr, cb, ce = out[f"{side}_chunk_row"], out[f"{side}_chunk_begin"], out[f"{side}_chunk_end"]
        part = np.full(cr.size, -1)
        for i in range(n):
            a, b = ptr[i], ptr[i + 1]
            assert np.array_equal(np.sort(key[a:b]), np.sort(orig[a:b]))
            if thr > 0 and deg[i] > thr:
                res = key[a:b] % 8
                assert np.all(np.diff(res) >= 0)
                for p in range(8):      # stable: each group keeps the original order
                    assert np.array_equal(key[a:b][res == p], orig[a:b][orig[a:b] % 8 == p])
            else:
                assert np.array_equal(key[a:b], orig[a:b])
        for c in range(cr.size):
            assert cb[c] < ce[c] <= cb[c] + chunk
            i = cr[c]
            assert ptr[i] <= cb[c] and ce[c] <= ptr[i + 1]
            if thr > 0 and deg[i] > thr:
                res = np.unique(key[cb[c]:ce[c]] % 8)
                assert res.size == 1
                part[c] = res[0]
        hub = out[f"{side}_hub"]
        assert np.array_equal(np.sort(hub), np.flatnonzero(deg > thr) if thr > 0 else hub)
        sched = out[f"{side}_sched"]
        if not np.any(part >= 0):
            assert sched.size == 0
            continue
        assert sched.size % 32 == 0
        assert np.array_equal(np.sort(sched[sched >= 0]), np.arange(cr.size))
        for p in range(8):
            slots = np.flatnonzero(np.isin(sched, np.flatnonzero(part == p)))
            assert np.all((slots // 4) % 8 == p)
            sizes = (ce - cb)[sched[slots]]
            assert np.all(np.diff(sizes) <= 0)
    colptr, rowidx = P.transpose(ip, out["indices"])
    assert np.array_equal(out["colptr"], colptr)
