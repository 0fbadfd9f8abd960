"""Pins of the fp64 oracle's backward (dot score).

* hand-derived closed forms (tests/golden/worked_example.json),
* central finite differences of the oracle's own forward (loss = <out, dOut>),
* torch fp64 autograd through dense masked attention (boolean / log-count mask),
* invariants: sum_j dK_j = 0 per head, sum_j dV_j = sum of dOut over non-empty rows,
  dQ = 0 on single-neighbour rows and on rows whose neighbour keys are all equal,
* agreement of the CSR-scatter, CSC-gather, sampled and per-row training-step forms, and
  of the row-pass / column-pass halves run over blocks of rows and columns.
"""
import json
import os

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A


def _graph(seed, n, m):
    rng = np.random.default_rng(seed)
    ip, ix = gg.random_multigraph(n, m, rng)
    return rng, ip, ix


def test_worked_example_backward(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    arr = lambda key: np.array(g[key], dtype=np.float64)
    ip = np.array(g["indptr"], np.int32)
    ix = np.array(g["indices"], np.int32)
    dq, dk, dv = A.backward(ip, ix, arr("q"), arr("k"), arr("v"), arr("dout"), g["scale"])
    ex = g["expected"]
    np.testing.assert_allclose(dq, np.array(ex["dq"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, np.array(ex["dk"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, np.array(ex["dv"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_central_finite_differences(seed):
    rng, ip, ix = _graph(seed, 9, 30)
    H, d = 2, 3
    q, k, v, do = (rng.standard_normal((9, H, d)) for _ in range(4))
    scale = 0.61
    dq, dk, dv = A.backward(ip, ix, q, k, v, do, scale)

    def loss(q_, k_, v_):
        out, _ = A.forward(ip, ix, q_, k_, v_, "dot", scale)
        return float((out * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                        loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


def _torch_dense_grads(ip, ix, q, k, v, do, scale):
    n = ip.size - 1
    c = np.zeros((n, n))
    np.add.at(c, (np.repeat(np.arange(n), np.diff(ip)), ix), 1.0)
    add = torch.from_numpy(np.where(c > 0, np.log(np.maximum(c, 1)), -np.inf))
    T = lambda x: torch.from_numpy(x).permute(1, 0, 2).contiguous().requires_grad_(True)
    tq, tk, tv = T(q), T(k), T(v)
    S = scale * torch.matmul(tq, tk.transpose(1, 2).contiguous()) + add  # [H, n, n]
    has = torch.from_numpy(c.sum(1) > 0)
    P = torch.softmax(S[:, has], dim=-1)
    out = torch.zeros(q.shape[1], n, q.shape[2], dtype=torch.float64)
    out[:, has] = torch.matmul(P, tv)
    (out * torch.from_numpy(do).permute(1, 0, 2)).sum().backward()
    back = lambda t: t.grad.permute(1, 0, 2).numpy()
    return back(tq), back(tk), back(tv)


@pytest.mark.parametrize("seed", [3, 4])
def test_backward_matches_torch_autograd_dense(seed):
    rng, ip, ix = _graph(seed, 30, 400)
    # one empty row
    dst = np.repeat(np.arange(30), np.diff(ip))
    ip, ix = gg.csr_from_edges(30, ix[dst != 4], dst[dst != 4])
    H, d = 3, 4
    q, k, v, do = (rng.standard_normal((30, H, d)) for _ in range(4))
    dq, dk, dv = A.backward(ip, ix, q, k, v, do, 0.5)
    rq, rk, rv = _torch_dense_grads(ip, ix, q, k, v, do, 0.5)
    np.testing.assert_allclose(dq, rq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, rk, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, rv, rtol=1e-11, atol=1e-12)


def test_gradient_invariants():
    rng, ip, ix = _graph(5, 80, 900)
    n, H, d = 80, 4, 8
    q, k, v, do = (rng.standard_normal((n, H, d)) for _ in range(4))
    dq, dk, dv = A.backward(ip, ix, q, k, v, do, None)
    # shifting every key by a constant vector shifts a row's scores uniformly
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    nonempty = np.diff(ip) > 0
    np.testing.assert_allclose(dv.sum(axis=0), do[nonempty].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_dq_vanishes_on_single_neighbour_and_equal_key_rows():
    rng = np.random.default_rng(6)
    n, H, d = 30, 2, 5
    src = np.r_[rng.integers(0, n, n), [0, 1, 2]]
    dst = np.r_[np.arange(n), [3, 3, 3]]         # row 3 gets 4 neighbours
    ip, ix = gg.csr_from_edges(n, src, dst)
    q, k, v, do = (rng.standard_normal((n, H, d)) for _ in range(4))
    k[ix[ip[3]:ip[4]]] = k[0]                    # all of row 3's keys equal
    dq, _, _ = A.backward(ip, ix, q, k, v, do, None)
    single = np.flatnonzero(np.diff(ip) == 1)
    assert single.size > 10
    assert np.all(dq[single] == 0.0)
    np.testing.assert_allclose(dq[3], 0.0, atol=1e-14)


def test_formulations_agree():
    rng, ip, ix = _graph(7, 60, 700)
    n, H, d = 60, 2, 6
    q, k, v, do = (rng.standard_normal((n, H, d)) for _ in range(4))
    a = A.backward(ip, ix, q, k, v, do, None)
    b = A.backward_by_columns(ip, ix, q, k, v, do, None)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
    rows = np.arange(n)
    out, lse, dq, cols, dkp, dvp = A.train_step_rows(ip, ix, q, k, v, do, rows, None)
    fo, fl = A.forward(ip, ix, q, k, v, "dot", None)
    np.testing.assert_allclose(out, fo, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dq, a[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dkp, a[1][cols], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dvp, a[2][cols], rtol=1e-12, atol=1e-12)
    sel = rng.choice(n, 12, replace=False)
    np.testing.assert_allclose(A.grad_q_rows(ip, ix, q, k, v, do, sel, None), a[0][sel],
                               rtol=1e-12, atol=1e-12)
    gk, gv = A.grad_kv_cols(ip, ix, q, k, v, do, sel, None)
    np.testing.assert_allclose(gk, a[1][sel], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gv, a[2][sel], rtol=1e-12, atol=1e-12)


def test_gat_scale_is_a_temperature():
    """LeakyReLU is positively homogeneous, so scale * LeakyReLU(s + t) equals the score
    of (scale * s, scale * t) at scale 1."""
    rng, ip, ix = _graph(8, 40, 300)
    s, t = rng.standard_normal((40, 2)), rng.standard_normal((40, 2))
    v = rng.standard_normal((40, 2, 3))
    a, la = A.forward(ip, ix, s, t, v, "gat", 2.5, 0.2)
    b, lb = A.forward(ip, ix, 2.5 * s, 2.5 * t, v, "gat", 1.0, 0.2)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ GAT-style backward

def _gat_inputs(seed, n, m, H=2, d=3):
    rng, ip, ix = _graph(seed, n, m)
    s, t = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    v, do = rng.standard_normal((n, H, d)), rng.standard_normal((n, H, d))
    return ip, ix, s, t, v, do


@pytest.mark.parametrize("seed", [0, 1])
def test_gat_backward_matches_central_finite_differences(seed):
    ip, ix, s, t, v, do = _gat_inputs(seed, 9, 30)
    scale, a = 1.3, 0.2
    ds, dt, dv = A.backward_gat(ip, ix, s, t, v, do, scale, a)

    def loss(s_, t_, v_):
        out, _ = A.forward(ip, ix, s_, t_, v_, "gat", scale, a)
        return float((out * do).sum())

    h = 1e-6
    for name, x, g in (("s", s, ds), ("t", t, dt), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            ap = {"s": s, "t": t, "v": v}; ap[name] = xp
            am = {"s": s, "t": t, "v": v}; am[name] = xm
            num[idx] = (loss(ap["s"], ap["t"], ap["v"]) - loss(am["s"], am["t"], am["v"])) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_gat_backward_matches_torch_autograd_dense():
    ip, ix, s, t, v, do = _gat_inputs(5, 30, 400, H=3, d=4)
    n, H = 30, 3
    dst = np.repeat(np.arange(n), np.diff(ip))
    ip, ix = gg.csr_from_edges(n, ix[dst != 6], dst[dst != 6])          # row 6 empty
    ds, dt, dv = A.backward_gat(ip, ix, s, t, v, do, 0.9, 0.1)
    c = np.zeros((n, n))
    np.add.at(c, (np.repeat(np.arange(n), np.diff(ip)), ix), 1.0)
    add = torch.from_numpy(np.where(c > 0, np.log(np.maximum(c, 1)), -np.inf))
    ts = torch.from_numpy(s.T.copy()).requires_grad_(True)           # [H, n]
    tt = torch.from_numpy(t.T.copy()).requires_grad_(True)
    tv = torch.from_numpy(v).permute(1, 0, 2).contiguous().requires_grad_(True)
    x = ts[:, :, None] + tt[:, None, :]
    S = 0.9 * torch.nn.functional.leaky_relu(x, 0.1) + add
    has = torch.from_numpy(c.sum(1) > 0)
    P = torch.softmax(S[:, has], dim=-1)
    out = torch.zeros(H, n, 4, dtype=torch.float64)
    out[:, has] = torch.matmul(P, tv)
    (out * torch.from_numpy(do).permute(1, 0, 2)).sum().backward()
    np.testing.assert_allclose(ds, ts.grad.T.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dt, tt.grad.T.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_gat_backward_linear_regime_closed_forms():
    """With every s_i + t_j >= 0 the score is scale (s_i + t_j): each row's softmax ignores
    s_i (ds = 0), and shifting every t by a constant shifts rows uniformly (sum dt = 0)."""
    ip, ix, s, t, v, do = _gat_inputs(7, 50, 500, H=3, d=4)
    s = s + 50.0
    ds, dt, dv = A.backward_gat(ip, ix, s, t, v, do, 1.0, 0.2)
    np.testing.assert_allclose(ds, 0.0, atol=1e-12)
    np.testing.assert_allclose(dt.sum(axis=0), 0.0, atol=1e-12)
    nonempty = np.diff(ip) > 0
    np.testing.assert_allclose(dv.sum(axis=0), do[nonempty].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_gat_backward_sampled_forms_agree():
    ip, ix, s, t, v, do = _gat_inputs(8, 70, 800, H=2, d=5)
    ds, dt, dv = A.backward_gat(ip, ix, s, t, v, do, 1.0, 0.2)
    rng = np.random.default_rng(0)
    sel = rng.choice(70, 15, replace=False)
    np.testing.assert_allclose(A.grad_s_rows(ip, ix, s, t, v, do, sel, 1.0, 0.2), ds[sel],
                               rtol=1e-12, atol=1e-13)
    gt, gv = A.grad_tv_cols(ip, ix, s, t, v, do, sel, 1.0, 0.2)
    np.testing.assert_allclose(gt, dt[sel], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gv, dv[sel], rtol=1e-12, atol=1e-13)


def test_train_step_rows_gat_is_the_plain_step():
    """The GAT per-row training step over all rows is forward + backward_gat; over a subset
    it gives those rows' outputs and ds, and two disjoint subsets' dt / dv shares add up to
    the whole."""
    rng = np.random.default_rng(17)
    n, H, d = 40, 3, 5
    ip, ix = gg.random_multigraph(n, 300, rng, hub_rows=(3,), hub_deg=60)
    s_, t_ = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    v, do = rng.standard_normal((n, H, d)), rng.standard_normal((n, H, d))
    out, lse = A.forward(ip, ix, s_, t_, v, "gat", 0.7, 0.15)
    ds, dt, dv = A.backward_gat(ip, ix, s_, t_, v, do, 0.7, 0.15)
    o2, l2, ds2, cols, dt2, dv2 = A.train_step_rows_gat(ip, ix, s_, t_, v, do, np.arange(n),
                                                        0.7, 0.15)
    np.testing.assert_allclose(o2, out, atol=1e-13)
    np.testing.assert_allclose(l2, lse, atol=1e-13)
    np.testing.assert_allclose(ds2, ds, atol=1e-12)
    full_t, full_v = np.zeros_like(dt), np.zeros_like(dv)
    full_t[cols], full_v[cols] = dt2, dv2
    np.testing.assert_allclose(full_t, dt, atol=1e-12)
    np.testing.assert_allclose(full_v, dv, atol=1e-12)
    a, b = np.arange(0, n, 2), np.arange(1, n, 2)
    acc_t, acc_v = np.zeros_like(dt), np.zeros_like(dv)
    for rows in (a, b):
        o3, _, ds3, c3, dt3, dv3 = A.train_step_rows_gat(ip, ix, s_, t_, v, do, rows, 0.7, 0.15)
        np.testing.assert_allclose(o3, out[rows], atol=1e-13)
        np.testing.assert_allclose(ds3, ds[rows], atol=1e-12)
        np.add.at(acc_t, c3, dt3)
        np.add.at(acc_v, c3, dv3)
    np.testing.assert_allclose(acc_t, dt, atol=1e-12)
    np.testing.assert_allclose(acc_v, dv, atol=1e-12)


@pytest.mark.parametrize("seed", [31, 32])
def test_row_and_column_passes_in_blocks_are_the_plain_step(seed):
    """The halves the full-size parity runs in worker blocks: rows in contiguous blocks
    give out, lse, dq and every edge's (alpha, dS) at its CSR position; columns in blocks
    give dk, dv. Composed they equal forward + backward (pinned above), with an empty row
    and an empty column in the graph."""
    rng = np.random.default_rng(seed)
    n, H, d = 70, 3, 5
    ip, ix = gg.random_multigraph(n, 900, rng, self_loops=False, hub_rows=(4,), hub_deg=120)
    keep = (np.repeat(np.arange(n), np.diff(ip)) != 9) & (ix != 11)   # row 9, column 11 empty
    dst = np.repeat(np.arange(n), np.diff(ip))[keep]
    ip, ix = gg.csr_from_edges(n, ix[keep], dst)
    q, k, v, do = (rng.standard_normal((n, H, d)) for _ in range(4))
    fo, fl = A.forward(ip, ix, q, k, v, "dot", None)
    dq0, dk0, dv0 = A.backward(ip, ix, q, k, v, do, None)
    E = ix.size
    ea, ed = np.full((E, H), np.nan), np.full((E, H), np.nan)
    cuts = np.unique(np.r_[0, rng.choice(n, 6), n])
    for r0, r1 in zip(cuts[:-1], cuts[1:]):
        out, lse, dq, a, s = A.row_pass(ip, ix, q, k, v, do, np.arange(r0, r1), None)
        np.testing.assert_allclose(out, fo[r0:r1], rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(fl[r0:r1]))
        np.testing.assert_allclose(lse[~np.isneginf(lse)], fl[r0:r1][~np.isneginf(lse)],
                                   rtol=1e-13)
        np.testing.assert_allclose(dq, dq0[r0:r1], rtol=1e-12, atol=1e-12)
        ea[ip[r0]:ip[r1]], ed[ip[r0]:ip[r1]] = a, s
    assert not np.isnan(ea).any() and not np.isnan(ed).any()     # every edge written once
    np.testing.assert_allclose(ea[ip[4]:ip[5]].sum(axis=0), 1.0, rtol=1e-13)   # row 4's weights
    order, col_start, edge_row = A.transpose_order(ip, ix)
    assert np.array_equal(np.sort(ix[order], kind="stable"), ix[order])
    for c0, c1 in ((0, 23), (23, 24), (24, n)):
        dk, dv = A.column_pass(q, do, ea, ed, order, col_start, edge_row, np.arange(c0, c1))
        np.testing.assert_allclose(dk, dk0[c0:c1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv, dv0[c0:c1], rtol=1e-12, atol=1e-12)
    assert np.all(dk0[11] == 0) and np.all(dq0[9] == 0)


def _blocky_graph(seed, n=70):
    rng = np.random.default_rng(seed)
    ip, ix = gg.random_multigraph(n, 900, rng, self_loops=False, hub_rows=(4,), hub_deg=120)
    dst = np.repeat(np.arange(n), np.diff(ip))
    keep = (dst != 9) & (ix != 11)                      # row 9 and column 11 empty
    ip, ix = gg.csr_from_edges(n, ix[keep], dst[keep])
    return rng, ip, ix


@pytest.mark.parametrize("slope", [0.2, -0.3])
def test_gat_row_and_column_passes_in_blocks_are_the_plain_step(slope):
    """The GAT-style halves run over random blocks of rows and columns reproduce forward
    and backward_gat (pinned above by finite differences and dense autograd)."""
    rng, ip, ix = _blocky_graph(33)
    n, H, d = 70, 3, 5
    s, t = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    v, do = rng.standard_normal((n, H, d)), rng.standard_normal((n, H, d))
    fo, fl = A.forward(ip, ix, s, t, v, "gat", 1.3, slope)
    ds0, dt0, dv0 = A.backward_gat(ip, ix, s, t, v, do, 1.3, slope)
    ea, ed = np.full((ix.size, H), np.nan), np.full((ix.size, H), np.nan)
    cuts = np.unique(np.r_[0, rng.choice(n, 5), n])
    for r0, r1 in zip(cuts[:-1], cuts[1:]):
        out, lse, ds, a, e = A.row_pass_gat(ip, ix, s, t, v, do, np.arange(r0, r1), 1.3, slope)
        np.testing.assert_allclose(out, fo[r0:r1], rtol=1e-13, atol=1e-14)
        fin = ~np.isneginf(fl[r0:r1])
        np.testing.assert_array_equal(np.isneginf(lse), ~fin)
        np.testing.assert_allclose(lse[fin], fl[r0:r1][fin], rtol=1e-13)
        np.testing.assert_allclose(ds, ds0[r0:r1], rtol=1e-12, atol=1e-12)
        ea[ip[r0]:ip[r1]], ed[ip[r0]:ip[r1]] = a, e
    assert not np.isnan(ea).any() and not np.isnan(ed).any()
    order, col_start, edge_row = A.transpose_order(ip, ix)
    for c0, c1 in ((0, 11), (11, 12), (12, n)):
        dt, dv = A.column_pass_gat(s, t, do, ea, ed, order, col_start, edge_row,
                                   np.arange(c0, c1), 1.3, slope)
        np.testing.assert_allclose(dt, dt0[c0:c1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv, dv0[c0:c1], rtol=1e-12, atol=1e-12)
    assert np.all(dt0[11] == 0) and np.all(ds0[9] == 0)
