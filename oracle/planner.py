"""Reference degree-binning planner and CSC transpose (numpy).  Test infrastructure only.

What a plan holds (the library's C++ planner must produce identical arrays):

Row bins by in-degree deg_i = indptr[i+1] - indptr[i] (the pages' degree-aware tiling,
"On Efficient Scaling of GNNs via IO-Aware Layers Implementations", Technical Summary >
Methodology: nodes split by a degree threshold into light and heavy sets, heavy ones
processed as parallel edge chunks; here with a middle bin):
    light   deg <= T_L             (includes deg 0)
    medium  T_L < deg <= T_H
    hub     deg > T_H
Each bin lists its rows by degree descending, ties by ascending id.
Hub row i is cut into chunks [indptr[i] + kC, min(indptr[i] + (k+1)C, indptr[i+1])),
listed hub by hub in hub-bin order; hub_chunk_ptr[h] is the first chunk of the h-th hub.

Optional XCD split (a layout choice for a GPU with 8 L2 partitions, not from the pages):
with a split threshold T_X > 0, rows with deg > T_X are hubs too, their CSR entries are
regrouped stably by source id mod 8 (group p holds the sources j with j mod 8 = p, in CSR
order), and each nonempty group is chunked on its own, groups in order p = 0..7. The
chunk schedule then deals chunks to dispatch slots: partition p's chunks (unsplit hubs'
chunks are dealt to partitions 0, 1, ..., 7, 0, ... in chunk order) sorted by length
descending, ties by chunk id, the k-th to slot ((k // 4) * 8 + p) * 4 + k % 4; unused slots
hold -1. The schedule is empty when no row is split. Split columns are regrouped by
destination id mod 8 the same way, csc_rel moving with rowidx.

Cached transpose (Methodology: precomputed transposed adjacency for the backward):
colptr[j] = number of edges with source < j; rowidx lists, per source column j, the
destination of every edge i -> j, destinations ascending, duplicates kept.  Column bins
and column chunks follow the same rules on out-degree.
"""
from __future__ import annotations

import numpy as np

__all__ = ["validate_csr", "bin_rows", "chunk_hubs", "xcd_schedule", "transpose", "plan"]


def validate_csr(indptr, indices) -> bool:
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    n = indptr.size - 1
    if n < 0 or indptr[0] != 0 or indptr[-1] != indices.size:
        return False
    if np.any(np.diff(indptr) < 0):
        return False
    return indices.size == 0 or (indices.min() >= 0 and indices.max() < n)


XCDS = 8          # L2 partitions of the GPU
SLOT_BLOCK = 4    # dispatch slots (wavefronts) per workgroup


def bin_rows(deg, t_light, t_hub, t_split=0):
    deg = np.asarray(deg, dtype=np.int64)
    ids = np.arange(deg.size, dtype=np.int64)
    order = np.lexsort((ids, -deg))            # degree descending, then id ascending
    d = deg[order]
    heavy = (d > t_hub) | ((t_split > 0) & (d > t_split))
    light = order[d <= t_light]
    medium = order[(d > t_light) & ~heavy]
    hub = order[(d > t_light) & heavy]
    return light.astype(np.int32), medium.astype(np.int32), hub.astype(np.int32)


def chunk_hubs(ptr, hub, chunk, keys=None, t_split=0, comp=None):
    """Hub chunks, and each chunk's partition (-1 unless split). Split hubs regroup
    ``keys`` (and ``comp`` alongside) in place."""
    ptr = np.asarray(ptr, dtype=np.int64)
    rows, begins, ends, part, first = [], [], [], [], [0]

    def cut(i, b, e, p):
        for s in range(b, e, chunk):
            rows.append(int(i))
            begins.append(s)
            ends.append(min(s + chunk, e))
            part.append(p)

    for i in hub:
        b, e = int(ptr[i]), int(ptr[i + 1])
        if t_split > 0 and e - b > t_split:
            seg = keys[b:e].copy()
            o = np.argsort(seg % XCDS, kind="stable")
            keys[b:e] = seg[o]
            if comp is not None:
                comp[b:e] = comp[b:e][o]
            edges = b + np.r_[0, np.cumsum(np.bincount(seg % XCDS, minlength=XCDS))]
            for p in range(XCDS):
                cut(i, int(edges[p]), int(edges[p + 1]), p)
        else:
            cut(i, b, e, -1)
        first.append(len(rows))
    as32 = lambda x: np.asarray(x, dtype=np.int32)
    return as32(rows), as32(begins), as32(ends), as32(first), np.asarray(part, np.int64)


def xcd_schedule(begins, ends, part):
    """Dispatch slot -> chunk id (-1 = unused); empty when no chunk has a partition."""
    part = np.asarray(part, np.int64)
    if not np.any(part >= 0):
        return np.zeros(0, np.int32)
    queues = [[] for _ in range(XCDS)]
    turn = 0
    for c, p in enumerate(part.tolist()):
        if p < 0:
            p = turn % XCDS
            turn += 1
        queues[p].append(c)
    size = (np.asarray(ends, np.int64) - np.asarray(begins, np.int64)).tolist()
    queues = [sorted(q, key=lambda c: -size[c]) for q in queues]  # stable: ties by id
    blocks = max((len(q) + SLOT_BLOCK - 1) // SLOT_BLOCK for q in queues)
    sched = np.full(blocks * XCDS * SLOT_BLOCK, -1, np.int32)
    for p, q in enumerate(queues):
        for k, c in enumerate(q):
            sched[((k // SLOT_BLOCK) * XCDS + p) * SLOT_BLOCK + k % SLOT_BLOCK] = c
    return sched


def transpose(indptr, indices):
    """(colptr [N+1], rowidx [E]) of the CSR, destinations ascending within a column."""
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    n = indptr.size - 1
    edge_row = np.repeat(np.arange(n, dtype=np.int64), np.diff(indptr))
    order = np.argsort(indices, kind="stable")
    colptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(np.bincount(indices, minlength=n), out=colptr[1:])
    return colptr.astype(np.int32), edge_row[order].astype(np.int32)


def transpose_positions(indptr, indices):
    """For each transpose entry (in transpose order), the position of that edge within its
    CSR row: the CSR edges listed column by column, then k - indptr[row(k)]."""
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    k = np.arange(indices.size, dtype=np.int64)
    row = np.repeat(np.arange(indptr.size - 1, dtype=np.int64), np.diff(indptr))
    order = np.argsort(indices, kind="stable")
    return (k - indptr[row])[order].astype(np.int32)


def plan(indptr, indices, light_max_deg=16, hub_min_deg_exclusive=1024, hub_chunk=1024,
         build_csc=True, col_hub_min_deg_exclusive=None, col_hub_chunk=None, xcd_split=0,
         col_xcd_split=None):
    """All plan arrays as a dict of int32 arrays (names match the library's export)."""
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.array(indices, dtype=np.int64)          # the plan's own (regrouped) copy
    out = {}
    deg = np.diff(indptr)
    out["row_light"], out["row_medium"], out["row_hub"] = bin_rows(
        deg, light_max_deg, hub_min_deg_exclusive, xcd_split)
    (out["row_chunk_row"], out["row_chunk_begin"], out["row_chunk_end"],
     out["row_hub_chunk_ptr"], part) = chunk_hubs(indptr, out["row_hub"], hub_chunk, indices,
                                                   xcd_split)
    out["row_sched"] = xcd_schedule(out["row_chunk_begin"], out["row_chunk_end"], part)
    out["indptr"] = indptr.astype(np.int32)
    out["indices"] = indices.astype(np.int32)
    if build_csc:
        colptr, rowidx = transpose(indptr, indices)
        rel = transpose_positions(indptr, indices)
        odeg = np.diff(colptr.astype(np.int64))
        cth = hub_min_deg_exclusive if col_hub_min_deg_exclusive is None \
            else col_hub_min_deg_exclusive
        cch = hub_chunk if col_hub_chunk is None else col_hub_chunk
        cxs = xcd_split if col_xcd_split is None else col_xcd_split
        out["col_light"], out["col_medium"], out["col_hub"] = bin_rows(
            odeg, light_max_deg, cth, cxs)
        rowidx = rowidx.astype(np.int64)
        (out["col_chunk_row"], out["col_chunk_begin"], out["col_chunk_end"],
         out["col_hub_chunk_ptr"], cpart) = chunk_hubs(colptr, out["col_hub"], cch, rowidx,
                                                        cxs, rel)
        out["col_sched"] = xcd_schedule(out["col_chunk_begin"], out["col_chunk_end"], cpart)
        out["colptr"], out["rowidx"], out["csc_rel"] = colptr, rowidx.astype(np.int32), rel
    return out
