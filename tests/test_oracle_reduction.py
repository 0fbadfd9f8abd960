"""Pins of the reduction oracle (min / max neighbourhood pooling, its arg and the routed
gradient) against things other than itself: a hand-derived worked example, torch's
scatter_reduce, a sequential brute-force scan, invariants, central finite differences
and torch autograd."""
import json
import os
import math

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import planner as P
from oracle import reduction as R


def _f(v):
    return float(v) if not isinstance(v, str) else {"-inf": -math.inf, "-0.0": -0.0}[v]


def _load_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "reduction_example.json")))
    x = np.array([[_f(v) for v in row] for row in g["x"]])
    return g, np.array(g["indptr"]), np.array(g["indices"]), x, np.array(g["dout"])


@pytest.mark.parametrize("op", ["max", "min"])
def test_worked_example(golden_dir, op):
    g, ip, ix, x, dout = _load_golden(golden_dir)
    exp = g["expected"][op]
    out, arg = R.reduce_forward(ip, ix, x, op)
    want = np.array([[_f(v) for v in row] for row in exp["out"]])
    assert np.array_equal(arg, np.array(exp["arg"]))
    assert np.array_equal(out, want)
    assert np.array_equal(np.signbit(out), np.signbit(want))     # zero signs as derived
    dx = R.reduce_backward(arg, dout, g["n_nodes"])
    assert np.array_equal(dx, np.array(exp["dx"], dtype=float))
    assert np.array_equal(R.reduce_backward_by_columns(ip, ix, arg, dout), dx)


def _graph(seed, n=40, m=300, loops=True):
    rng = np.random.default_rng(seed)
    ip, ix = gg.random_multigraph(n, m, rng, self_loops=loops)
    return rng, ip, ix


@pytest.mark.parametrize("op,name", [("max", "amax"), ("min", "amin")])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_values_match_torch_scatter_reduce(op, name, seed):
    rng, ip, ix = _graph(seed, m=80, loops=False)   # sparse: some rows are empty
    x = rng.standard_normal((40, 6))
    out, arg = R.reduce_forward(ip, ix, x, op)
    dst = torch.from_numpy(np.repeat(np.arange(40), np.diff(ip)))
    src = torch.from_numpy(np.asarray(ix, dtype=np.int64))
    ref = torch.zeros(40, 6, dtype=torch.float64).scatter_reduce(
        0, dst[:, None].expand(-1, 6), torch.from_numpy(x)[src], reduce=name,
        include_self=False)
    assert np.array_equal(out, ref.numpy())
    empty = np.diff(ip) == 0
    assert empty.any() and (arg[empty] == -1).all() and (out[empty] == 0).all()


def _scan(ip, ix, x, op):
    """Brute force: visit every neighbour in CSR order, one element at a time, keeping
    the best (value, id) with plain comparisons."""
    N, F = len(ip) - 1, x.shape[1]
    out = np.zeros((N, F))
    arg = np.full((N, F), -1)
    for i in range(N):
        for c in range(F):
            best, bid = None, None
            for j in ix[ip[i]:ip[i + 1]]:
                v = x[j, c]
                if best is None:
                    best, bid = v, j
                    continue
                wins = v > best if op == "max" else v < best
                if wins or (v == best and j < bid):
                    best, bid = v, j
            if bid is not None:
                out[i, c], arg[i, c] = best, bid
    return out, arg


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("seed", [3, 4])
def test_ties_match_brute_force_scan(op, seed):
    # values on a coarse grid and graph rows in random order: many ties, so the
    # smallest-id rule decides most args
    rng, ip, ix = _graph(seed, n=30, m=400, loops=False)
    ix = ix.copy()
    for i in range(30):
        rng.shuffle(ix[ip[i]:ip[i + 1]])
    x = rng.integers(-3, 4, size=(30, 5)).astype(float)
    out, arg = R.reduce_forward(ip, ix, x, op)
    o2, a2 = _scan(ip, ix, x, op)
    assert np.array_equal(arg, a2) and np.array_equal(out, o2)


@pytest.mark.parametrize("op", ["max", "min"])
def test_invariants(op):
    rng, ip, ix = _graph(5, n=50, m=500)
    xb = gg.f32_to_bf16_bits(rng.standard_normal((50, 2, 8)).astype(np.float32))
    x = gg.bf16_bits_to_f32(xb).astype(np.float64).reshape(50, -1)
    out, arg = R.reduce_forward(ip, ix, xb, op)          # bf16 bits in, widened exactly
    F = x.shape[1]
    for i in range(50):
        J = ix[ip[i]:ip[i + 1]]
        assert np.isin(arg[i], J).all()                          # the arg is a neighbour
        assert np.array_equal(out[i], x[arg[i], np.arange(F)])   # out = x at the arg
        if op == "max":
            assert (out[i][None] >= x[J]).all()
        else:
            assert (out[i][None] <= x[J]).all()
    # min is max of the negation, with the same ids (the tie rule is on ids only)
    o_neg, a_neg = R.reduce_forward(ip, ix, -x, "max" if op == "min" else "min")
    assert np.array_equal(a_neg, arg) and np.array_equal(-o_neg, out)
    # neighbour order within a row changes nothing, bit for bit
    ix2 = ix.copy()
    for i in range(50):
        rng.shuffle(ix2[ip[i]:ip[i + 1]])
    o3, a3 = R.reduce_forward(ip, ix2, x, op)
    assert np.array_equal(a3, arg) and np.array_equal(o3, out)
    # chunk partials merged as (value, index) pairs in any order give the same result
    o4, a4 = R.reduce_forward_chunked(ip, ix, x, op, np.random.default_rng(1))
    assert np.array_equal(a4, arg) and np.array_equal(o4, out)


def test_single_neighbour_rows_copy_the_source():
    ip = np.array([0, 1, 2, 3])
    ix = np.array([2, 0, 0])
    x = np.array([[1.5, -2.0], [9.0, 9.0], [-0.0, 3.0]])
    for op in ("max", "min"):
        out, arg = R.reduce_forward(ip, ix, x, op)
        assert np.array_equal(arg, [[2, 2], [0, 0], [0, 0]])
        assert np.array_equal(out, x[[2, 0, 0]]) and np.signbit(out[0, 0])


def test_merge_pairs_rules():
    v, i = R.merge_pairs([1.0, 2.0, 3.0, 0.0], [5, 5, 5, -1], [1.0, 2.5, 2.0, -7.0],
                         [4, 6, 1, 9], "max")
    assert np.array_equal(v, [1.0, 2.5, 3.0, -7.0]) and np.array_equal(i, [4, 6, 5, 9])
    v, i = R.merge_pairs([1.0, 0.0], [5, 3], [9.0, 0.0], [-1, -1], "min")
    assert np.array_equal(i, [5, 3])                   # an empty partial never wins


@pytest.mark.parametrize("op", ["max", "min"])
def test_backward_matches_finite_differences(op):
    rng, ip, ix = _graph(6, n=20, m=120, loops=False)
    x = rng.standard_normal((20, 4))        # continuous values: no ties
    w = rng.standard_normal((20, 4))
    _, arg = R.reduce_forward(ip, ix, x, op)
    dx = R.reduce_backward(arg, w, 20)
    h = 1e-6
    num = np.zeros_like(x)
    for j in range(20):
        for c in range(4):
            xp, xm = x.copy(), x.copy()
            xp[j, c] += h
            xm[j, c] -= h
            num[j, c] = ((R.reduce_forward(ip, ix, xp, op)[0] * w).sum()
                         - (R.reduce_forward(ip, ix, xm, op)[0] * w).sum()) / (2 * h)
    np.testing.assert_allclose(dx, num, rtol=0, atol=1e-8)


@pytest.mark.parametrize("op,name", [("max", "amax"), ("min", "amin")])
def test_backward_matches_torch_autograd(op, name):
    rng, ip, ix = _graph(7, n=30, m=300)
    x = rng.standard_normal((30, 5))
    w = rng.standard_normal((30, 5))
    _, arg = R.reduce_forward(ip, ix, x, op)
    tx = torch.from_numpy(x.copy()).requires_grad_(True)
    dst = torch.from_numpy(np.repeat(np.arange(30), np.diff(ip)))
    src = torch.from_numpy(np.asarray(ix, dtype=np.int64))
    # torch routes the gradient along the gathered copies; a parallel edge is two copies
    # of one x_j holding the same value (a tie that torch splits between them), and the
    # gradient of x_j is the sum over its copies, i.e. dout once
    y = torch.zeros(30, 5, dtype=torch.float64).scatter_reduce(
        0, dst[:, None].expand(-1, 5), tx[src], reduce=name, include_self=False)
    (y * torch.from_numpy(w)).sum().backward()
    np.testing.assert_allclose(R.reduce_backward(arg, w, 30), tx.grad.numpy(), rtol=0,
                               atol=1e-12)


def test_backward_invariants_and_parallel_edges():
    rng, ip, ix = _graph(8, n=25, m=400)      # dense enough for many parallel edges
    assert any(len(set(ix[ip[i]:ip[i + 1]])) < ip[i + 1] - ip[i] for i in range(25))
    x = gg.bf16_bits_to_f32(gg.f32_to_bf16_bits(
        rng.standard_normal((25, 6)).astype(np.float32))).astype(np.float64)
    dout = rng.standard_normal((25, 6))
    for op in ("max", "min"):
        _, arg = R.reduce_forward(ip, ix, x, op)
        dx = R.reduce_backward(arg, dout, 25)
        # every (row, element) routes its gradient to exactly one source
        np.testing.assert_allclose(dx.sum(0), dout[np.diff(ip) > 0].sum(0), atol=1e-12)
        # the column formulation (each distinct destination once) agrees
        np.testing.assert_allclose(R.reduce_backward_by_columns(ip, ix, arg, dout), dx,
                                   rtol=1e-13, atol=1e-13)
        colptr, rowidx = P.transpose(ip, ix)
        cols = [0, 7, 13]
        d2, rows, arg_rows = R.grad_cols_sampled(ip, ix, colptr, rowidx, x, dout, cols, op)
        np.testing.assert_allclose(d2, dx[cols], rtol=1e-13, atol=1e-13)
        assert np.array_equal(arg_rows, arg[rows])


def test_nan_is_rejected():
    with pytest.raises(ValueError):
        R.reduce_forward(np.array([0, 1]), np.array([0]), np.array([[math.nan]]))


def test_train_step_rows_is_the_row_share_of_the_backward():
    rng, ip, ix = _graph(9, n=30, m=200)
    x = rng.standard_normal((30, 4))
    dout = rng.standard_normal((30, 4))
    rows = np.array([1, 4, 5, 17, 29])
    out, arg, ids, dxi = R.train_step_rows(ip, ix, x, dout, rows, "max")
    full_out, full_arg = R.reduce_forward(ip, ix, x, "max")
    assert np.array_equal(out, full_out[rows]) and np.array_equal(arg, full_arg[rows])
    masked = np.full_like(full_arg, -1)
    masked[rows] = full_arg[rows]
    dx = R.reduce_backward(masked, dout, 30)
    assert np.array_equal(dx[ids], dxi) and not np.delete(dx, ids, axis=0).any()


def test_slots_point_at_the_first_edge_of_the_winner():
    rng, ip, ix = _graph(10, n=40, m=900)        # many parallel edges
    ix = ix.copy()
    for i in range(40):
        rng.shuffle(ix[ip[i]:ip[i + 1]])
    x = rng.integers(-2, 3, size=(40, 6)).astype(float)
    _, arg = R.reduce_forward(ip, ix, x, "min")
    sl = R.slots_of(ip, ix, np.arange(40), arg)
    for i in range(40):
        J = ix[ip[i]:ip[i + 1]]
        for c in range(6):
            k = sl[i, c]
            assert J[k] == arg[i, c] and not (J[:k] == arg[i, c]).any()
    e_ip = np.array([0, 0, 2]); e_ix = np.array([0, 0])
    _, a2 = R.reduce_forward(e_ip, e_ix, np.ones((2, 3)), "max")
    assert np.array_equal(R.slots_of(e_ip, e_ix, [0, 1], a2), [[-1] * 3, [0] * 3])
