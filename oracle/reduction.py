"""fp64 oracle of the degree-aware neighbourhood reduction (min / max pooling).

Test infrastructure only (see the package docstring).

Definition followed: "On Efficient Scaling of GNNs via IO-Aware Layers
Implementations", Technical Summary > Methodology: the reduction-based family is a
per-edge computation followed by a neighbourhood-wise reduction such as min or max
pooling, and the heavy-row partial results are combined as (value, index) pairs.  The
pages print no formula; the plainest reading, used here, takes the message of edge
(i <- j) to be the source row x_j itself and reduces every feature element separately:

    out[i, c] = max_{j in J_i} x[j, c]        (or min)
    arg[i, c] = the source id j that attains it

with J_i = indices[indptr[i]:indptr[i+1]] (CSR row = destination).  When several
neighbours attain the extreme the smallest source id wins, a rule that does not depend on
the order of a row's neighbours, so the index result is unique.  Values compare as
numbers (-0 equals +0); out[i, c] is x[arg[i, c], c] as stored.  A row with no
neighbours gives out = 0 and arg = -1.  Inputs are finite or infinite, never NaN.

The compact form of arg used by the backward, slot[i, c], is the position within row i
(k - indptr[i]) of the first edge of that row coming from arg[i, c]; -1 for an empty row.

Backward (the gradient of a max/min is routed to the element that attained it):
    dx[arg[i, c], c] += dout[i, c]    for every row i with arg[i, c] >= 0
A parallel edge (j listed twice in a row) is one variable x_j, so it receives the
gradient once.

All arithmetic is fp64; bf16 inputs arrive as uint16 bit patterns and are widened
exactly (comparisons of widened values are the comparisons of the stored values).
"""
from __future__ import annotations

import numpy as np

from .attention import widen

__all__ = ["EMPTY_ARG", "reduce_rows", "reduce_forward", "merge_pairs",
           "reduce_forward_chunked", "reduce_backward", "reduce_backward_by_columns",
           "reduce_backward_cols", "grad_cols_sampled", "train_step_rows", "slots_of"]

EMPTY_ARG = -1


def _features(x) -> np.ndarray:
    xf = widen(x)
    xf = xf.reshape(xf.shape[0], -1)
    if np.isnan(xf).any():
        raise ValueError("reduction oracle: NaN inputs are outside the definition")
    return xf


def _extreme(vals: np.ndarray, ids: np.ndarray, op: str):
    """Per column of vals [k, F]: the extreme value and the smallest id attaining it."""
    m = vals.max(axis=0) if op == "max" else vals.min(axis=0)
    big = np.iinfo(np.int64).max
    arg = np.where(vals == m[None, :], ids[:, None], big).min(axis=0)
    return m, arg


def reduce_rows(indptr, indices, x, rows, op="max"):
    """out, arg for the listed rows (fp64 [len(rows), F], int64 [len(rows), F]).  Only
    the neighbour rows of the listed rows are read (and widened)."""
    assert op in ("max", "min")
    x = np.asarray(x)
    F = int(np.prod(x.shape[1:]))
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, F))
    arg = np.full((rows.size, F), EMPTY_ARG, dtype=np.int64)
    for n, i in enumerate(rows):
        J = np.asarray(indices[indptr[i]:indptr[i + 1]], dtype=np.int64)
        if J.size == 0:
            continue
        xj = _features(x[J])
        _, a = _extreme(xj, J, op)
        arg[n] = a
        # the stored value of the winner (keeps the sign of a zero): the first position
        # in the row that holds the winning id
        pos = (J[:, None] == a[None, :]).argmax(axis=0)
        out[n] = xj[pos, np.arange(F)]
    return out, arg


def reduce_forward(indptr, indices, x, op="max"):
    N = len(indptr) - 1
    return reduce_rows(indptr, indices, x, np.arange(N), op)


def merge_pairs(va, ia, vb, ib, op="max"):
    """Combine two partial (value, index) results elementwise: the better value wins, an
    equal value goes to the smaller index; index EMPTY_ARG marks an empty partial."""
    va, vb = np.asarray(va, np.float64), np.asarray(vb, np.float64)
    ia, ib = np.asarray(ia, np.int64), np.asarray(ib, np.int64)
    better = (vb > va) if op == "max" else (vb < va)
    take_b = (ia == EMPTY_ARG) | ((ib != EMPTY_ARG) & (better | ((vb == va) & (ib < ia))))
    return np.where(take_b, vb, va), np.where(take_b, ib, ia)


def reduce_forward_chunked(indptr, indices, x, op="max", rng=None, max_chunk=4):
    """The same reduction computed per random edge chunk of each row and combined with
    merge_pairs in a shuffled order: the heavy-row scheme of the pages (chunk partials
    merged as (value, index) pairs).  Must equal reduce_forward exactly."""
    rng = np.random.default_rng(0) if rng is None else rng
    xf = _features(x)
    N, F = len(indptr) - 1, xf.shape[1]
    out = np.zeros((N, F))
    arg = np.full((N, F), EMPTY_ARG, dtype=np.int64)
    for i in range(N):
        b, e = int(indptr[i]), int(indptr[i + 1])
        cuts = [b]
        while cuts[-1] < e:
            cuts.append(min(e, cuts[-1] + int(rng.integers(1, max_chunk + 1))))
        parts = []
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            J = np.asarray(indices[c0:c1], dtype=np.int64)
            m, a = _extreme(xf[J], J, op)
            parts.append((m, a))
        rng.shuffle(parts)
        v, a = np.zeros(F), np.full(F, EMPTY_ARG, dtype=np.int64)
        for m, p in parts:
            v, a = merge_pairs(v, a, m, p, op)
        out[i] = np.where(a >= 0, xf[np.maximum(a, 0), np.arange(F)], 0.0)
        arg[i] = a
    return out, arg


def reduce_backward(arg, dout, n_nodes):
    """dx [n_nodes, F] from the forward's arg and the output gradient (scatter form)."""
    dof = widen(dout).reshape(np.asarray(arg).shape[0], -1)
    arg = np.asarray(arg, dtype=np.int64).reshape(dof.shape)
    dx = np.zeros((n_nodes, dof.shape[1]))
    rows, cols = np.nonzero(arg >= 0)
    np.add.at(dx, (arg[rows, cols], cols), dof[rows, cols])
    return dx


def reduce_backward_cols(colptr, rowidx, arg, dout, cols):
    """dx for the listed source nodes, gathered over the destinations that list them in
    the transpose (colptr, rowidx), each distinct destination once: the column
    formulation of reduce_backward."""
    dof = widen(dout).reshape(np.asarray(arg).shape[0], -1)
    arg = np.asarray(arg, dtype=np.int64).reshape(dof.shape)
    out = np.zeros((len(cols), dof.shape[1]))
    for n, j in enumerate(cols):
        for i in np.unique(np.asarray(rowidx[colptr[j]:colptr[j + 1]], dtype=np.int64)):
            hit = arg[i] == j
            out[n][hit] += dof[i][hit]
    return out


def reduce_backward_by_columns(indptr, indices, arg, dout):
    from .planner import transpose
    colptr, rowidx = transpose(indptr, indices)
    N = len(indptr) - 1
    return reduce_backward_cols(colptr, rowidx, arg, dout, np.arange(N))


def grad_cols_sampled(indptr, indices, colptr, rowidx, x, dout, cols, op="max"):
    """dx for a few source nodes of a large graph: the forward's arg of every destination
    that lists them is computed here (reduce_rows), then the column formulation.  Returns
    (dx [len(cols), F], rows, arg_rows) so the caller can also compare those args."""
    rows = np.unique(np.concatenate(
        [np.asarray(rowidx[colptr[j]:colptr[j + 1]], dtype=np.int64) for j in cols]
        + [np.zeros(0, np.int64)]))
    _, arg_rows = reduce_rows(indptr, indices, x, rows, op)
    dout = np.asarray(dout)
    pos = {int(i): n for n, i in enumerate(rows)}
    out = np.zeros((len(cols), arg_rows.shape[1]))
    for n, j in enumerate(cols):
        for i in np.unique(np.asarray(rowidx[colptr[j]:colptr[j + 1]], dtype=np.int64)):
            hit = arg_rows[pos[int(i)]] == j
            out[n][hit] += widen(dout[i]).reshape(-1)[hit]
    return out, rows, arg_rows


def train_step_rows(indptr, indices, x, dout, rows, op="max"):
    """Forward of the listed rows and their share of the backward: the gradient they
    route, returned compressed as (ids, dx_ids) with dx_ids[k] the contribution to
    dx[ids[k]] (so a sample of rows needs no [N, F] array)."""
    out, arg = reduce_rows(indptr, indices, x, rows, op)
    dof = np.stack([widen(dout[i]).reshape(-1) for i in rows]) if len(rows) else \
        np.zeros((0, arg.shape[1]))
    ids, local = np.unique(arg[arg >= 0], return_inverse=True)
    dx_ids = np.zeros((ids.size, arg.shape[1]))
    r, c = np.nonzero(arg >= 0)
    np.add.at(dx_ids, (local, c), dof[r, c])
    return out, arg, ids, dx_ids


def slots_of(indptr, indices, rows, arg_rows):
    """slot of the listed rows given their arg: the position within the row of the first
    edge from the winning id (-1 where arg is -1)."""
    arg_rows = np.asarray(arg_rows, dtype=np.int64)
    out = np.full(arg_rows.shape, -1, dtype=np.int64)
    for n, i in enumerate(np.asarray(rows, dtype=np.int64)):
        J = np.asarray(indices[indptr[i]:indptr[i + 1]], dtype=np.int64)
        a = arg_rows[n]
        if J.size == 0:
            continue
        first = (J[:, None] == a[None, :]).argmax(axis=0)
        out[n] = np.where(a >= 0, first, -1)
    return out
