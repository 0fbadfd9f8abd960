"""fp64 oracle of fused CSR graph attention (forward and recompute backward).

Test infrastructure only (see the package docstring).

Definition followed: "On Efficient Scaling of GNNs via IO-Aware Layers
Implementations", Technical Summary > Methodology, attention-based layers.  For every
destination node i of a CSR graph and every head h:

    e_k   = score(i, J_k)                      over the neighbour multiset J of row i
    alpha = softmax_k(e)                       (two passes: max, then exp / sum)
    out_i = sum_k alpha_k v_{J_k}
    lse_i = max_k e_k + ln sum_k exp(e_k - max)

Score forms (the pages name Graph Transformer and GAT-style layers but print no
formula; these are the standard definitions):
    dot:  e = scale * <q_i, k_j>               (scale = 1/sqrt(d) unless given)
    gat:  e = scale * LeakyReLU_a(s_i + t_j)   (per-node, per-head scalars; scale = 1)

The backward (Methodology, "Backward Pass": cached per-node log-sum-exp, weights
recomputed) is written out from the chain rule of the same definition, row by row:
    dp_k  = <dOut_i, v_{J_k}>,  D = sum_k alpha_k dp_k,  dS_k = alpha_k (dp_k - D)
    dq_i  = scale sum_k dS_k k_{J_k};  dk_{J_k} += scale dS_k q_i;  dv_{J_k} += alpha_k dOut_i

GAT-style backward, x_ij = s_i + t_j, LeakyReLU'(x) = 1 for x >= 0 else neg_slope (the
branch the forward takes at 0), same dS:
    ds_i += scale dS_ij LeakyReLU'(x_ij);  dt_j += scale dS_ij LeakyReLU'(x_ij);
    dv_j += alpha_ij dOut_i

GATv2 score (Brody et al., the GATv2 the pages name; destination projection xd, source
projection xs, which is also the message, attention vector a [H, d]):
    z_ij = xd_i + xs_j,  e_ij = scale * sum_c a[h,c] LeakyReLU(z_ij[h,c]),
    out_i = sum_j softmax_j(e)_ij xs_j
Its backward, with g = LeakyReLU'(z) elementwise and dS as above (dp_ij = <dOut_i, xs_j>):
    dxd_i += scale dS_ij (a * g_ij);  dxs_j += scale dS_ij (a * g_ij) + alpha_ij dOut_i;
    da    += scale dS_ij LeakyReLU(z_ij)   (summed over every edge)

Conventions: CSR row = destination; parallel edges count with multiplicity; a row with
no neighbours gives out = 0 and lse = -inf and no gradient.  All arithmetic is fp64;
bf16 inputs arrive as uint16 bit patterns and are widened exactly.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "leaky_relu", "row_scores", "row_softmax", "forward_rows", "forward",
    "backward", "backward_by_columns", "grad_q_rows", "grad_kv_cols", "train_step_rows",
    "backward_gat", "grad_s_rows", "grad_tv_cols", "gatv2_row_scores", "forward_gatv2",
    "forward_gatv2_rows", "backward_gatv2", "grad_gatv2_rows", "grad_gatv2_cols",
    "train_step_rows_gatv2", "forward_online_chunked", "train_step_rows_gat", "row_pass",
    "transpose_order", "column_pass", "row_pass_gat", "column_pass_gat", "row_pass_gatv2",
    "column_pass_gatv2",
]


def widen(x) -> np.ndarray:
    """Exact fp64 value of a stored tensor: float arrays as-is, uint16 = bf16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def leaky_relu(x: np.ndarray, neg_slope: float) -> np.ndarray:
    return np.where(x >= 0.0, x, neg_slope * x)


def _neighbours(indptr, indices, i):
    return indices[int(indptr[i]):int(indptr[i + 1])]


def row_scores(i, indptr, indices, a, b, score="dot", scale=None, neg_slope=0.2):
    """Scores e[k, h] of row i, materialised ([deg, H], fp64).

    dot: a = q [N,H,d], b = k [N,H,d].   gat: a = s [N,H], b = t [N,H].
    ``scale`` and ``neg_slope`` are used at their given (fp32) values, widened.
    """
    J = _neighbours(indptr, indices, i)
    if score == "dot":
        qi = widen(a[i])                       # [H, d]
        kj = widen(b[J])                       # [deg, H, d]
        if scale is None:
            scale = 1.0 / np.sqrt(qi.shape[-1])
        return float(scale) * np.einsum("hc,khc->kh", qi, kj)
    if score == "gat":
        si = widen(a[i])                       # [H]
        tj = widen(b[J])                       # [deg, H]
        sc = 1.0 if scale is None else float(scale)
        return sc * leaky_relu(si[None, :] + tj, float(neg_slope))
    raise ValueError(score)


def row_softmax(e: np.ndarray):
    """Two-pass softmax over axis 0 of e [deg, H]: returns (alpha, lse)."""
    m = e.max(axis=0)
    w = np.exp(e - m[None, :])
    l = w.sum(axis=0)
    return w / l[None, :], m + np.log(l)


def forward_rows(indptr, indices, a, b, v, rows, score="dot", scale=None, neg_slope=0.2):
    """out [R, H, d] and lse [R, H] (fp64) for the listed rows."""
    rows = np.asarray(rows, dtype=np.int64)
    H, d = v.shape[1], v.shape[2]
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    for r, i in enumerate(rows):
        J = _neighbours(indptr, indices, i)
        if J.size == 0:
            continue
        e = row_scores(i, indptr, indices, a, b, score, scale, neg_slope)
        alpha, lse[r] = row_softmax(e)
        out[r] = np.einsum("kh,khc->hc", alpha, widen(v[J]))
    return out, lse


def forward(indptr, indices, a, b, v, score="dot", scale=None, neg_slope=0.2):
    n = indptr.size - 1
    return forward_rows(indptr, indices, a, b, v, np.arange(n), score, scale, neg_slope)


def _merge_states(x, y):
    """Combine two running softmax states (m [H], l [H], acc [H, d]) over disjoint edge
    sets: rescale both to the larger maximum and add. An empty state has m = -inf."""
    (ma, la, aa), (mb, lb, ab) = x, y
    m = np.maximum(ma, mb)
    fa = np.where(np.isneginf(ma), 0.0, np.exp(ma - np.where(np.isneginf(m), 0.0, m)))
    fb = np.where(np.isneginf(mb), 0.0, np.exp(mb - np.where(np.isneginf(m), 0.0, m)))
    return m, la * fa + lb * fb, aa * fa[:, None] + ab * fb[:, None]


def forward_online_chunked(indptr, indices, a, b, v, rng, score="dot", scale=None,
                           neg_slope=0.2, max_chunk=None):
    """The streaming form of the same forward ("On Efficient Scaling of GNNs via IO-Aware
    Layers Implementations", Technical Summary > Methodology, attention-based layers,
    forward pass: online softmax keeping running statistics instead of edge-wise logits).
    Each row's edges are cut at random boundaries into chunks (at most max_chunk edges,
    default: random lengths up to the degree); each chunk streams its edges one by one
    into a running state (m = max score so far, l = sum of exp(e - m), acc = sum of
    exp(e - m) v), starting empty; the chunk states are then merged in ascending order and
    out = acc / l, lse = m + ln l. Exactly the two-pass softmax up to rounding; test pin
    only (the hub-chunk partials and their ordered merge compute this)."""
    n = indptr.size - 1
    H, d = v.shape[1], v.shape[2]
    out = np.zeros((n, H, d))
    lse = np.full((n, H), -np.inf)
    vf = widen(v)
    empty = lambda: (np.full(H, -np.inf), np.zeros(H), np.zeros((H, d)))
    for i in range(n):
        J = _neighbours(indptr, indices, i)
        if J.size == 0:
            continue
        e = row_scores(i, indptr, indices, a, b, score, scale, neg_slope)   # [deg, H]
        cuts, pos = [0], 0
        while pos < J.size:
            pos += int(rng.integers(1, (max_chunk or J.size) + 1))
            cuts.append(min(pos, J.size))
        total = empty()
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            m, l, acc = empty()
            for k in range(c0, c1):                     # one edge at a time
                m_new = np.maximum(m, e[k])
                f = np.exp(m - m_new)                   # 0 while the state is empty
                w = np.exp(e[k] - m_new)
                l = l * f + w
                acc = acc * f[:, None] + w[:, None] * vf[J[k]]
                m = m_new
            total = _merge_states(total, (m, l, acc))
        m, l, acc = total
        out[i] = acc / l[:, None]
        lse[i] = m + np.log(l)
    return out, lse


def _row_backward(i, indptr, indices, q, k, v, dout, scale):
    """Per-row pieces of the dot-score backward: (J, alpha [deg,H], dS [deg,H])."""
    J = _neighbours(indptr, indices, i)
    e = row_scores(i, indptr, indices, q, k, "dot", scale)
    alpha, _ = row_softmax(e)
    dp = np.einsum("hc,khc->kh", widen(dout[i]), widen(v[J]))
    D = (alpha * dp).sum(axis=0)
    return J, alpha, alpha * (dp - D[None, :])


def _scale_of(q, scale):
    return 1.0 / np.sqrt(q.shape[-1]) if scale is None else float(scale)


def backward(indptr, indices, q, k, v, dout, scale=None):
    """dq, dk, dv [N, H, d] (fp64) by rows, scattering dK/dV in CSR order."""
    sc = _scale_of(q, scale)
    n = indptr.size - 1
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for i in range(n):
        if indptr[i + 1] == indptr[i]:
            continue
        J, alpha, dS = _row_backward(i, indptr, indices, q, k, v, dout, sc)
        dq[i] = sc * np.einsum("kh,khc->hc", dS, widen(k[J]))
        np.add.at(dk, J, sc * dS[:, :, None] * widen(q[i])[None])
        np.add.at(dv, J, alpha[:, :, None] * widen(dout[i])[None])
    return dq, dk, dv


def backward_by_columns(indptr, indices, q, k, v, dout, scale=None):
    """Same gradients, but dK/dV gathered per source column (a CSC-ordered formulation
    with its own transpose), dQ per row.  Agrees with ``backward`` to rounding."""
    sc = _scale_of(q, scale)
    n = indptr.size - 1
    deg = np.diff(indptr)
    edge_row = np.repeat(np.arange(n), deg)
    dS_all = np.zeros((indices.size, q.shape[1]))
    al_all = np.zeros((indices.size, q.shape[1]))
    dq = np.zeros(q.shape)
    for i in range(n):
        if deg[i] == 0:
            continue
        J, alpha, dS = _row_backward(i, indptr, indices, q, k, v, dout, sc)
        dq[i] = sc * np.einsum("kh,khc->hc", dS, widen(k[J]))
        dS_all[indptr[i]:indptr[i + 1]] = dS
        al_all[indptr[i]:indptr[i + 1]] = alpha
    order = np.argsort(indices, kind="stable")
    col_start = np.searchsorted(indices[order], np.arange(n + 1))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for j in range(n):
        es = order[col_start[j]:col_start[j + 1]]
        if es.size == 0:
            continue
        rows = edge_row[es]
        dk[j] = sc * np.einsum("eh,ehc->hc", dS_all[es], widen(q[rows]))
        dv[j] = np.einsum("eh,ehc->hc", al_all[es], widen(dout[rows]))
    return dq, dk, dv


def grad_q_rows(indptr, indices, q, k, v, dout, rows, scale=None):
    """dq [R, H, d] for the listed rows only."""
    sc = _scale_of(q, scale)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size,) + tuple(q.shape[1:]))
    for r, i in enumerate(rows):
        if indptr[i + 1] == indptr[i]:
            continue
        J, _, dS = _row_backward(i, indptr, indices, q, k, v, dout, sc)
        dq[r] = sc * np.einsum("kh,khc->hc", dS, widen(k[J]))
    return dq


def grad_kv_cols(indptr, indices, q, k, v, dout, cols, scale=None):
    """dk, dv [C, H, d] for the listed source columns only: every edge (i -> j) with j in
    ``cols`` contributes its row's dS and alpha."""
    sc = _scale_of(q, scale)
    cols = np.asarray(cols, dtype=np.int64)
    slot = {int(j): c for c, j in enumerate(cols)}
    dk = np.zeros((cols.size,) + tuple(k.shape[1:]))
    dv = np.zeros((cols.size,) + tuple(v.shape[1:]))
    pos = np.flatnonzero(np.isin(indices, cols))
    rows = np.searchsorted(indptr, pos, side="right") - 1
    for i in np.unique(rows):
        J, alpha, dS = _row_backward(i, indptr, indices, q, k, v, dout, sc)
        qi, doi = widen(q[i]), widen(dout[i])
        for kk in np.flatnonzero(np.isin(J, cols)):
            c = slot[int(J[kk])]
            dk[c] += sc * dS[kk][:, None] * qi
            dv[c] += alpha[kk][:, None] * doi
    return dk, dv


def train_step_rows(indptr, indices, q, k, v, dout, rows, scale=None):
    """Forward and backward of the listed rows, each row's work done once.

    Returns (out [R,H,d], lse [R,H], dq [R,H,d], cols, dk_part [C,H,d], dv_part [C,H,d])
    where ``cols`` are the source columns the rows touch (ascending) and dk_part/dv_part
    hold those rows' contributions to dK/dV.  With rows = all rows this is exactly
    ``forward`` plus ``backward``.
    """
    sc = _scale_of(q, scale)
    rows = np.asarray(rows, dtype=np.int64)
    H, d = q.shape[1], q.shape[2]
    segs = [indices[int(indptr[i]):int(indptr[i + 1])] for i in rows]
    cols = np.unique(np.concatenate(segs)) if segs else np.zeros(0, np.int64)
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    dq = np.zeros((rows.size, H, d))
    dk = np.zeros((cols.size, H, d))
    dv = np.zeros((cols.size, H, d))
    for r, i in enumerate(rows):
        J = segs[r]
        if J.size == 0:
            continue
        e = row_scores(i, indptr, indices, q, k, "dot", sc)
        alpha, lse[r] = row_softmax(e)
        vj, kj = widen(v[J]), widen(k[J])
        out[r] = np.einsum("kh,khc->hc", alpha, vj)
        dp = np.einsum("hc,khc->kh", widen(dout[i]), vj)
        D = (alpha * dp).sum(axis=0)
        dS = alpha * (dp - D[None, :])
        dq[r] = sc * np.einsum("kh,khc->hc", dS, kj)
        slot = np.searchsorted(cols, J)
        np.add.at(dk, slot, sc * dS[:, :, None] * widen(q[i])[None])
        np.add.at(dv, slot, alpha[:, :, None] * widen(dout[i])[None])
    return out, lse, dq, cols, dk, dv


def row_pass(indptr, indices, q, k, v, dout, rows, scale=None):
    """The row half of the training step for the listed rows (the forward and the per-row
    loop of ``backward_by_columns``): out [R,H,d], lse [R,H] and dq [R,H,d] of each row,
    and the attention weight alpha [M,H] and score gradient dS [M,H] of each of its edges,
    the rows' edges concatenated in the order of ``rows`` (for a contiguous, ascending
    block of rows: the block's CSR positions).  With ``column_pass`` over every column this
    is ``forward`` plus ``backward``; the two halves let blocks of rows and of columns run
    apart."""
    sc = _scale_of(q, scale)
    rows = np.asarray(rows, dtype=np.int64)
    H, d = q.shape[1], q.shape[2]
    deg = (indptr[rows + 1] - indptr[rows]).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(deg)])
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    dq = np.zeros((rows.size, H, d))
    e_alpha = np.zeros((int(start[-1]), H))
    e_ds = np.zeros((int(start[-1]), H))
    for r, i in enumerate(rows):
        if deg[r] == 0:
            continue
        J = _neighbours(indptr, indices, i)
        e = row_scores(i, indptr, indices, q, k, "dot", sc)
        alpha, lse[r] = row_softmax(e)
        vj = widen(v[J])
        out[r] = np.einsum("kh,khc->hc", alpha, vj)
        dp = np.einsum("hc,khc->kh", widen(dout[i]), vj)
        D = (alpha * dp).sum(axis=0)
        dS = alpha * (dp - D[None, :])
        dq[r] = sc * np.einsum("kh,khc->hc", dS, widen(k[J]))
        e_alpha[start[r]:start[r + 1]] = alpha
        e_ds[start[r]:start[r + 1]] = dS
    return out, lse, dq, e_alpha, e_ds


def transpose_order(indptr, indices):
    """The transpose as a stable sort of CSR positions by source: (order, col_start,
    edge_row), where column j's edges are the CSR positions order[col_start[j]:
    col_start[j+1]] (destinations ascending) and edge_row[p] is the destination row of
    CSR position p."""
    n = indptr.size - 1
    order = np.argsort(indices, kind="stable")
    col_start = np.searchsorted(indices[order], np.arange(n + 1))
    edge_row = np.repeat(np.arange(n), np.diff(indptr))
    return order, col_start, edge_row


def column_pass(q, dout, e_alpha, e_ds, order, col_start, edge_row, cols, scale=None):
    """dk, dv [C,H,d] of the listed source columns from every edge's alpha and dS (indexed
    by CSR position, as ``row_pass`` gives them for all rows): for column j and each edge
    (i -> j), dk_j += scale dS q_i and dv_j += alpha dout_i (the per-column loop of
    ``backward_by_columns``)."""
    sc = _scale_of(q, scale)
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((cols.size,) + tuple(q.shape[1:]))
    dv = np.zeros((cols.size,) + tuple(dout.shape[1:]))
    for c, j in enumerate(cols):
        es = order[col_start[j]:col_start[j + 1]]
        if es.size == 0:
            continue
        rows = edge_row[es]
        dk[c] = sc * np.einsum("eh,ehc->hc", e_ds[es], widen(q[rows]))
        dv[c] = np.einsum("eh,ehc->hc", e_alpha[es], widen(dout[rows]))
    return dk, dv


def leaky_relu_grad(x: np.ndarray, neg_slope: float) -> np.ndarray:
    return np.where(x >= 0.0, 1.0, neg_slope)


def _row_backward_gat(i, indptr, indices, s, t, v, dout, scale, neg_slope):
    """Per-row pieces of the GAT-style backward: (J, alpha, dS, LeakyReLU'(x)) [deg, H]."""
    J = _neighbours(indptr, indices, i)
    e = row_scores(i, indptr, indices, s, t, "gat", scale, neg_slope)
    alpha, _ = row_softmax(e)
    dp = np.einsum("hc,khc->kh", widen(dout[i]), widen(v[J]))
    D = (alpha * dp).sum(axis=0)
    x = widen(s[i])[None, :] + widen(t[J])
    return J, alpha, alpha * (dp - D[None, :]), leaky_relu_grad(x, float(neg_slope))


def backward_gat(indptr, indices, s, t, v, dout, scale=1.0, neg_slope=0.2):
    """ds [N,H], dt [N,H], dv [N,H,d] (fp64) of the GAT-style layer, by rows with a
    sequential scatter into dt and dv."""
    sc = float(scale)
    n = indptr.size - 1
    ds = np.zeros(s.shape)
    dt = np.zeros(t.shape)
    dv = np.zeros(v.shape)
    for i in range(n):
        if indptr[i + 1] == indptr[i]:
            continue
        J, alpha, dS, g = _row_backward_gat(i, indptr, indices, s, t, v, dout, sc, neg_slope)
        ds[i] = sc * (dS * g).sum(axis=0)
        np.add.at(dt, J, sc * dS * g)
        np.add.at(dv, J, alpha[:, :, None] * widen(dout[i])[None])
    return ds, dt, dv


def train_step_rows_gat(indptr, indices, s, t, v, dout, rows, scale=1.0, neg_slope=0.2):
    """Forward and backward of the listed rows of the GAT-style layer, each row's work done
    once (the GAT counterpart of ``train_step_rows``).

    Returns (out [R,H,d], lse [R,H], ds [R,H], cols, dt_part [C,H], dv_part [C,H,d]):
    ``cols`` are the source columns the rows touch (ascending), and dt_part and dv_part
    hold those rows' contributions. With rows = all rows this is exactly ``forward``
    plus ``backward_gat``."""
    rows = np.asarray(rows, dtype=np.int64)
    H, d = v.shape[1], v.shape[2]
    segs = [indices[int(indptr[i]):int(indptr[i + 1])] for i in rows]
    cols = np.unique(np.concatenate(segs)) if segs else np.zeros(0, np.int64)
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    ds = np.zeros((rows.size, H))
    dt = np.zeros((cols.size, H))
    dv = np.zeros((cols.size, H, d))
    for r, i in enumerate(rows):
        J = segs[r]
        if J.size == 0:
            continue
        e = row_scores(i, indptr, indices, s, t, "gat", scale, neg_slope)
        alpha, lse[r] = row_softmax(e)
        vj = widen(v[J])
        out[r] = np.einsum("kh,khc->hc", alpha, vj)
        dp = np.einsum("hc,khc->kh", widen(dout[i]), vj)
        D = (alpha * dp).sum(axis=0)
        dS = alpha * (dp - D[None, :])
        g = leaky_relu_grad(widen(s[i])[None, :] + widen(t[J]), float(neg_slope))
        ds[r] = scale * (dS * g).sum(axis=0)
        slot = np.searchsorted(cols, J)
        np.add.at(dt, slot, scale * dS * g)
        np.add.at(dv, slot, alpha[:, :, None] * widen(dout[i])[None])
    return out, lse, ds, cols, dt, dv


def row_pass_gat(indptr, indices, s, t, v, dout, rows, scale=1.0, neg_slope=0.2):
    """The row half of the GAT-style training step for the listed rows: out [R,H,d],
    lse [R,H] and ds [R,H] of each row, and alpha [M,H] and dS [M,H] of each of its edges,
    the rows' edges concatenated in the order of ``rows``.  With ``column_pass_gat`` over
    every column this is ``forward`` plus ``backward_gat``."""
    sc = float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    H, d = v.shape[1], v.shape[2]
    deg = (indptr[rows + 1] - indptr[rows]).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(deg)])
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    ds = np.zeros((rows.size, H))
    e_alpha = np.zeros((int(start[-1]), H))
    e_ds = np.zeros((int(start[-1]), H))
    for r, i in enumerate(rows):
        if deg[r] == 0:
            continue
        J = _neighbours(indptr, indices, i)
        e = row_scores(i, indptr, indices, s, t, "gat", sc, neg_slope)
        alpha, lse[r] = row_softmax(e)
        vj = widen(v[J])
        out[r] = np.einsum("kh,khc->hc", alpha, vj)
        dp = np.einsum("hc,khc->kh", widen(dout[i]), vj)
        D = (alpha * dp).sum(axis=0)
        dS = alpha * (dp - D[None, :])
        g = leaky_relu_grad(widen(s[i])[None, :] + widen(t[J]), float(neg_slope))
        ds[r] = sc * (dS * g).sum(axis=0)
        e_alpha[start[r]:start[r + 1]] = alpha
        e_ds[start[r]:start[r + 1]] = dS
    return out, lse, ds, e_alpha, e_ds


def column_pass_gat(s, t, dout, e_alpha, e_ds, order, col_start, edge_row, cols, scale=1.0,
                    neg_slope=0.2):
    """dt [C,H] and dv [C,H,d] of the listed source columns from every edge's alpha and dS
    (by CSR position, over the transpose of ``transpose_order``): for column j and each
    edge (i -> j), dt_j += scale dS LeakyReLU'(s_i + t_j) and dv_j += alpha dout_i."""
    sc = float(scale)
    cols = np.asarray(cols, dtype=np.int64)
    dt = np.zeros((cols.size,) + tuple(t.shape[1:]))
    dv = np.zeros((cols.size,) + tuple(dout.shape[1:]))
    for c, j in enumerate(cols):
        es = order[col_start[j]:col_start[j + 1]]
        if es.size == 0:
            continue
        rows = edge_row[es]
        g = leaky_relu_grad(widen(s[rows]) + widen(t[j])[None, :], float(neg_slope))
        dt[c] = sc * (e_ds[es] * g).sum(axis=0)
        dv[c] = np.einsum("eh,ehc->hc", e_alpha[es], widen(dout[rows]))
    return dt, dv


def grad_s_rows(indptr, indices, s, t, v, dout, rows, scale=1.0, neg_slope=0.2):
    """ds [R, H] for the listed rows only."""
    sc = float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    ds = np.zeros((rows.size, s.shape[1]))
    for r, i in enumerate(rows):
        if indptr[i + 1] == indptr[i]:
            continue
        _, _, dS, g = _row_backward_gat(i, indptr, indices, s, t, v, dout, sc, neg_slope)
        ds[r] = sc * (dS * g).sum(axis=0)
    return ds


def grad_tv_cols(indptr, indices, s, t, v, dout, cols, scale=1.0, neg_slope=0.2):
    """dt [C, H] and dv [C, H, d] for the listed source columns only."""
    sc = float(scale)
    cols = np.asarray(cols, dtype=np.int64)
    slot = {int(j): c for c, j in enumerate(cols)}
    dt = np.zeros((cols.size, t.shape[1]))
    dv = np.zeros((cols.size,) + tuple(v.shape[1:]))
    pos = np.flatnonzero(np.isin(indices, cols))
    rows = np.searchsorted(indptr, pos, side="right") - 1
    for i in np.unique(rows):
        J, alpha, dS, g = _row_backward_gat(i, indptr, indices, s, t, v, dout, sc, neg_slope)
        doi = widen(dout[i])
        for kk in np.flatnonzero(np.isin(J, cols)):
            c = slot[int(J[kk])]
            dt[c] += sc * dS[kk] * g[kk]
            dv[c] += alpha[kk][:, None] * doi
    return dt, dv


# ----------------------------------------------------------------------------- GATv2

def gatv2_row_scores(i, indptr, indices, xd, xs, attn, scale=1.0, neg_slope=0.2):
    """e [deg, H] of row i: scale * sum_c a[h,c] LeakyReLU(xd[i,h,c] + xs[j,h,c])."""
    J = _neighbours(indptr, indices, i)
    z = widen(xd[i])[None] + widen(xs[J])                     # [deg, H, d]
    return float(scale) * np.einsum("hc,khc->kh", widen(attn), leaky_relu(z, float(neg_slope)))


def forward_gatv2_rows(indptr, indices, xd, xs, attn, rows, scale=1.0, neg_slope=0.2):
    rows = np.asarray(rows, dtype=np.int64)
    H, d = xs.shape[1], xs.shape[2]
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    for r, i in enumerate(rows):
        J = _neighbours(indptr, indices, i)
        if J.size == 0:
            continue
        alpha, lse[r] = row_softmax(gatv2_row_scores(i, indptr, indices, xd, xs, attn, scale,
                                                      neg_slope))
        out[r] = np.einsum("kh,khc->hc", alpha, widen(xs[J]))
    return out, lse


def forward_gatv2(indptr, indices, xd, xs, attn, scale=1.0, neg_slope=0.2):
    return forward_gatv2_rows(indptr, indices, xd, xs, attn, np.arange(indptr.size - 1), scale,
                              neg_slope)


def _row_backward_gatv2(i, indptr, indices, xd, xs, attn, dout, scale, neg_slope):
    """Per-row pieces: (J, alpha [deg,H], dS [deg,H], g [deg,H,d], lrelu(z) [deg,H,d])."""
    J = _neighbours(indptr, indices, i)
    z = widen(xd[i])[None] + widen(xs[J])
    lz = leaky_relu(z, float(neg_slope))
    e = float(scale) * np.einsum("hc,khc->kh", widen(attn), lz)
    alpha, _ = row_softmax(e)
    dp = np.einsum("hc,khc->kh", widen(dout[i]), widen(xs[J]))
    D = (alpha * dp).sum(axis=0)
    return J, alpha, alpha * (dp - D[None, :]), leaky_relu_grad(z, float(neg_slope)), lz


def train_step_rows_gatv2(indptr, indices, xd, xs, attn, dout, rows, scale=1.0, neg_slope=0.2):
    """GATv2 forward and backward of the listed rows, each row's work done once.

    Returns (out [R,H,d], lse [R,H], dxd [R,H,d], cols, dxs_part [C,H,d], dattn_part [H,d]):
    ``cols`` are the source columns the rows touch (ascending), dxs_part and dattn_part
    those rows' contributions.  With rows = all rows this is exactly ``forward_gatv2``
    plus ``backward_gatv2``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    H, d = xs.shape[1], xs.shape[2]
    segs = [np.asarray(indices[int(indptr[i]):int(indptr[i + 1])], dtype=np.int64) for i in rows]
    cols = np.unique(np.concatenate(segs)) if segs else np.zeros(0, np.int64)
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    dxd = np.zeros((rows.size, H, d))
    dxs = np.zeros((cols.size, H, d))
    da = np.zeros((H, d))
    a = widen(attn)
    for r, i in enumerate(rows):
        if segs[r].size == 0:
            continue
        e = gatv2_row_scores(i, indptr, indices, xd, xs, attn, scale, neg_slope)
        _, lse[r] = row_softmax(e)
        J, alpha, dS, g, lz = _row_backward_gatv2(i, indptr, indices, xd, xs, attn, dout,
                                                   scale, neg_slope)
        xsj = widen(xs[J])
        out[r] = np.einsum("kh,khc->hc", alpha, xsj)
        t = float(scale) * dS[:, :, None] * g * a[None]
        dxd[r] = t.sum(axis=0)
        slot = np.searchsorted(cols, J)
        np.add.at(dxs, slot, t + alpha[:, :, None] * widen(dout[i])[None])
        da += float(scale) * np.einsum("kh,khc->hc", dS, lz)
    return out, lse, dxd, cols, dxs, da


def backward_gatv2(indptr, indices, xd, xs, attn, dout, scale=1.0, neg_slope=0.2):
    """dxd, dxs [N,H,d] and dattn [H,d] (fp64), by rows with a sequential scatter."""
    sc = float(scale)
    a = widen(attn)
    n = indptr.size - 1
    dxd = np.zeros(xd.shape)
    dxs = np.zeros(xs.shape)
    da = np.zeros(attn.shape)
    for i in range(n):
        if indptr[i + 1] == indptr[i]:
            continue
        J, alpha, dS, g, lz = _row_backward_gatv2(i, indptr, indices, xd, xs, attn, dout, sc,
                                                  neg_slope)
        w = sc * dS[:, :, None] * g * a[None]                   # [deg, H, d]
        dxd[i] = w.sum(axis=0)
        np.add.at(dxs, J, w + alpha[:, :, None] * widen(dout[i])[None])
        da += sc * np.einsum("kh,khc->hc", dS, lz)
    return dxd, dxs, da


def row_pass_gatv2(indptr, indices, xd, xs, attn, dout, rows, scale=1.0, neg_slope=0.2):
    """The row half of the GATv2 training step for the listed rows: out [R,H,d], lse [R,H]
    and dxd [R,H,d] of each row, alpha [M,H] and dS [M,H] of each of its edges (the rows'
    edges concatenated in the order of ``rows``), and the rows' share of dattn [H,d].
    With ``column_pass_gatv2`` over every column this is ``forward_gatv2`` plus
    ``backward_gatv2`` (dattn = the sum of the shares)."""
    sc = float(scale)
    a = widen(attn)
    rows = np.asarray(rows, dtype=np.int64)
    H, d = xs.shape[1], xs.shape[2]
    deg = (indptr[rows + 1] - indptr[rows]).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(deg)])
    out = np.zeros((rows.size, H, d))
    lse = np.full((rows.size, H), -np.inf)
    dxd = np.zeros((rows.size, H, d))
    da = np.zeros((H, d))
    e_alpha = np.zeros((int(start[-1]), H))
    e_ds = np.zeros((int(start[-1]), H))
    for r, i in enumerate(rows):
        if deg[r] == 0:
            continue
        e = gatv2_row_scores(i, indptr, indices, xd, xs, attn, scale, neg_slope)
        _, lse[r] = row_softmax(e)
        J, alpha, dS, g, lz = _row_backward_gatv2(i, indptr, indices, xd, xs, attn, dout, sc,
                                                  neg_slope)
        out[r] = np.einsum("kh,khc->hc", alpha, widen(xs[J]))
        dxd[r] = (sc * dS[:, :, None] * g * a[None]).sum(axis=0)
        da += sc * np.einsum("kh,khc->hc", dS, lz)
        e_alpha[start[r]:start[r + 1]] = alpha
        e_ds[start[r]:start[r + 1]] = dS
    return out, lse, dxd, e_alpha, e_ds, da


def column_pass_gatv2(xd, xs, attn, dout, e_alpha, e_ds, order, col_start, edge_row, cols,
                      scale=1.0, neg_slope=0.2):
    """dxs [C,H,d] of the listed source columns from every edge's alpha and dS (by CSR
    position, over the transpose of ``transpose_order``): for column j and each edge
    (i -> j), dxs_j += scale dS (attn * LeakyReLU'(xd_i + xs_j)) + alpha dout_i."""
    sc = float(scale)
    a = widen(attn)
    cols = np.asarray(cols, dtype=np.int64)
    dxs = np.zeros((cols.size,) + tuple(xs.shape[1:]))
    for c, j in enumerate(cols):
        es = order[col_start[j]:col_start[j + 1]]
        if es.size == 0:
            continue
        rows = edge_row[es]
        g = leaky_relu_grad(widen(xd[rows]) + widen(xs[j])[None], float(neg_slope))
        dxs[c] = (sc * e_ds[es][:, :, None] * g * a[None]).sum(axis=0) + \
            np.einsum("eh,ehc->hc", e_alpha[es], widen(dout[rows]))
    return dxs


def grad_gatv2_rows(indptr, indices, xd, xs, attn, dout, rows, scale=1.0, neg_slope=0.2):
    """dxd [R,H,d] for the listed rows and those rows' contribution to dattn."""
    sc = float(scale)
    a = widen(attn)
    rows = np.asarray(rows, dtype=np.int64)
    dxd = np.zeros((rows.size,) + tuple(xd.shape[1:]))
    da = np.zeros(attn.shape)
    for r, i in enumerate(rows):
        if indptr[i + 1] == indptr[i]:
            continue
        _, _, dS, g, lz = _row_backward_gatv2(i, indptr, indices, xd, xs, attn, dout, sc,
                                              neg_slope)
        dxd[r] = (sc * dS[:, :, None] * g * a[None]).sum(axis=0)
        da += sc * np.einsum("kh,khc->hc", dS, lz)
    return dxd, da


def grad_gatv2_cols(indptr, indices, xd, xs, attn, dout, cols, scale=1.0, neg_slope=0.2):
    """dxs [C,H,d] for the listed source columns only."""
    sc = float(scale)
    a = widen(attn)
    cols = np.asarray(cols, dtype=np.int64)
    slot = {int(j): c for c, j in enumerate(cols)}
    dxs = np.zeros((cols.size,) + tuple(xs.shape[1:]))
    pos = np.flatnonzero(np.isin(indices, cols))
    rows = np.searchsorted(indptr, pos, side="right") - 1
    for i in np.unique(rows):
        J, alpha, dS, g, _ = _row_backward_gatv2(i, indptr, indices, xd, xs, attn, dout, sc,
                                                 neg_slope)
        doi = widen(dout[i])
        for kk in np.flatnonzero(np.isin(J, cols)):
            dxs[slot[int(J[kk])]] += sc * dS[kk][:, None] * g[kk] * a + alpha[kk][:, None] * doi
    return dxs
