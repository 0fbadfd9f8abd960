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

Cached transpose (Methodology: precomputed transposed adjacency for the backward):
colptr[j] = number of edges with source < j; rowidx lists, per source column j, the
destination of every edge i -> j, destinations ascending, duplicates kept.  Column bins
and column chunks follow the same rules on out-degree.
"""
from __future__ import annotations

import numpy as np

__all__ = ["validate_csr", "bin_rows", "chunk_hubs", "transpose", "plan"]


def validate_csr(indptr, indices) -> bool:
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    n = indptr.size - 1
    if n < 0 or indptr[0] != 0 or indptr[-1] != indices.size:
        return False
    if np.any(np.diff(indptr) < 0):
        return False
    return indices.size == 0 or (indices.min() >= 0 and indices.max() < n)


def bin_rows(deg, t_light, t_hub):
    deg = np.asarray(deg, dtype=np.int64)
    ids = np.arange(deg.size, dtype=np.int64)
    order = np.lexsort((ids, -deg))            # degree descending, then id ascending
    d = deg[order]
    light = order[d <= t_light]
    medium = order[(d > t_light) & (d <= t_hub)]
    hub = order[d > t_hub]
    return light.astype(np.int32), medium.astype(np.int32), hub.astype(np.int32)


def chunk_hubs(ptr, hub, chunk):
    ptr = np.asarray(ptr, dtype=np.int64)
    rows, begins, ends, first = [], [], [], [0]
    for i in hub:
        b, e = int(ptr[i]), int(ptr[i + 1])
        for s in range(b, e, chunk):
            rows.append(int(i))
            begins.append(s)
            ends.append(min(s + chunk, e))
        first.append(len(rows))
    as32 = lambda x: np.asarray(x, dtype=np.int32)
    return as32(rows), as32(begins), as32(ends), as32(first)


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
         build_csc=True, col_hub_min_deg_exclusive=None, col_hub_chunk=None):
    """All plan arrays as a dict of int32 arrays (names match the library's export)."""
    indptr = np.asarray(indptr, dtype=np.int64)
    out = {}
    deg = np.diff(indptr)
    out["row_light"], out["row_medium"], out["row_hub"] = bin_rows(
        deg, light_max_deg, hub_min_deg_exclusive)
    (out["row_chunk_row"], out["row_chunk_begin"], out["row_chunk_end"],
     out["row_hub_chunk_ptr"]) = chunk_hubs(indptr, out["row_hub"], hub_chunk)
    if build_csc:
        colptr, rowidx = transpose(indptr, indices)
        out["colptr"], out["rowidx"] = colptr, rowidx
        out["csc_rel"] = transpose_positions(indptr, indices)
        odeg = np.diff(colptr.astype(np.int64))
        cth = hub_min_deg_exclusive if col_hub_min_deg_exclusive is None \
            else col_hub_min_deg_exclusive
        cch = hub_chunk if col_hub_chunk is None else col_hub_chunk
        out["col_light"], out["col_medium"], out["col_hub"] = bin_rows(odeg, light_max_deg, cth)
        (out["col_chunk_row"], out["col_chunk_begin"], out["col_chunk_end"],
         out["col_hub_chunk_ptr"]) = chunk_hubs(colptr, out["col_hub"], cch)
    return out
