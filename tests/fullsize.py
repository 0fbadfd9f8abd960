"""Every-element parity at full workload sizes, on the host: the fp64 oracle over every
row (and every source column) of a workload, in forked worker processes, compared element
by element with the results a GPU run saved to a directory.

Run as a child process, ``python -m tests.fullsize SPEC.json``, from a GPU test: the
workers are forked from this fresh process, which never touches the GPU.  SPEC names the
workload, the GRAPHGEN_CACHE directory holding its generated inputs, the saved GPU
results (.npy: bf16 as uint16 bit patterns) and the checks to run; the child prints one
JSON line with, per tensor, the parity verdict and its statistics.

Criteria (the same as tests/gpu_util.py, applied to every element):
  fp32 inputs:  |x - r| <= max(1e-5, 1e-4 |r|)
  bf16 inputs:  |x - r| <= 2e-2 max(|r|, rms(r)), rms over the whole tensor
  lse:          |x - r| <= max(1e-5, 1e-4 |r|), -inf exactly where r = -inf
A worker cannot know the whole tensor's rms, so for bf16 it reports, over its elements,
the smallest rms under which all of them would pass (max of |x - r| / 2e-2 over the
elements with |x - r| > 2e-2 |r|); the tensor passes when that is at most its rms.
"""
from __future__ import annotations

import json
import mmap
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HOST_CPUS_PER_GPU = 16     # worker processes: at most the host CPUs allotted to each GPU

_G = {}                    # inputs and shared arrays, inherited by the forked workers


def workers() -> int:
    return max(1, min(HOST_CPUS_PER_GPU, len(os.sched_getaffinity(0))))


def shared_array(shape, dtype=np.float64):
    """A zeroed array in anonymous shared memory: writes by forked workers are seen by
    the parent and by the other workers."""
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    buf = mmap.mmap(-1, max(n, 1))
    return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(shape)


def balanced_blocks(ptr, k):
    """[lo, hi) ranges of rows (columns) of a CSR-like pointer array, about k of them, each
    with about the same number of edges plus rows."""
    n = ptr.size - 1
    if n == 0:
        return []
    work = ptr.astype(np.int64) + np.arange(n + 1)
    cuts = np.searchsorted(work, np.linspace(0, work[-1], k + 1), side="left")
    cuts[0], cuts[-1] = 0, n
    cuts = np.unique(cuts)
    return [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


# ----------------------------------------------------------------- per-block statistics

def stats(got, ref, kind, base=0):
    """Parity statistics of one block (flattened index base for the worst element)."""
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    st = {"n": int(ref.size), "nonfinite": 0, "sum_r2": 0.0, "sum_e2": 0.0, "max_err": 0.0,
          "need_rms": 0.0, "n_bad": 0, "ninf_mismatch": 0, "worst": None}
    if ref.size == 0:
        return st
    if kind == "lse":
        ninf = np.isneginf(ref)
        st["ninf_mismatch"] = int((np.isneginf(got) != ninf).sum())
        got, ref = got[~ninf], ref[~ninf]
        idx = np.flatnonzero(~ninf)
    else:
        idx = None
    fin = np.isfinite(got)
    st["nonfinite"] = int((~fin).sum())
    err = np.where(fin, np.abs(got - ref), np.inf)
    st["sum_r2"] = float(np.sum(ref * ref))
    st["sum_e2"] = float(np.sum(np.where(fin, err, 0.0) ** 2))
    st["max_err"] = float(err.max(initial=0.0))
    if kind == "bf16":
        over = err > 2e-2 * np.abs(ref)
        if over.any():
            need = np.where(over, err / 2e-2, 0.0)
            w = int(np.argmax(need))
            st["need_rms"] = float(need[w])
            st["worst"] = [base + w, float(got[w]), float(ref[w])]
    else:
        bound = np.maximum(1e-5, 1e-4 * np.abs(ref))
        bad = err > bound
        st["n_bad"] = int(bad.sum())
        if bad.any():
            w = int(np.argmax(err - bound))
            st["worst"] = [base + int(idx[w] if idx is not None else w), float(got[w]),
                           float(ref[w])]
    return st


def merge(parts, kind):
    """Tensor verdict from its blocks' statistics."""
    n = sum(p["n"] for p in parts)
    sum_r2 = sum(p["sum_r2"] for p in parts)
    rms = float(np.sqrt(sum_r2 / n)) if n else 0.0
    worst = [p["worst"] for p in parts if p["worst"] is not None]
    res = {"elements": n, "rms_ref": rms, "nonfinite": sum(p["nonfinite"] for p in parts),
           "max_abs_err": max((p["max_err"] for p in parts), default=0.0),
           "norm_rel_err": float(np.sqrt(sum(p["sum_e2"] for p in parts) / sum_r2))
           if sum_r2 else 0.0}
    if kind == "bf16":
        need = max((p["need_rms"] for p in parts), default=0.0)
        res["need_rms"] = need
        res["ok"] = res["nonfinite"] == 0 and need <= rms
    else:
        res["n_bad"] = sum(p["n_bad"] for p in parts)
        res["ninf_mismatch"] = sum(p["ninf_mismatch"] for p in parts)
        res["ok"] = res["nonfinite"] == 0 and res["n_bad"] == 0 and res["ninf_mismatch"] == 0
    if worst and not res["ok"]:
        res["worst"] = worst[:4]
    return res


# ----------------------------------------------------------------- worker tasks

def _rows_task(block):
    """Rows [r0, r1): the oracle's forward (and, for a training step, the row half of the
    backward, whose edge weights and score gradients go to the shared arrays), compared
    with the GPU's rows."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    g = _G
    r0, r1 = block
    rows = np.arange(r0, r1)
    ip, ix = g["ip"], g["ix"]
    res = {}
    with threadpool_limits(1):
        if g["train"]:
            out, lse, dq, ea, ed = A.row_pass(ip, ix, g["q"], g["k"], g["v"], g["dout"], rows,
                                              g["scale"])
            g["ea"][ip[r0]:ip[r1]] = ea
            g["ed"][ip[r0]:ip[r1]] = ed
        else:
            out, lse = A.forward_rows(ip, ix, g["q"], g["k"], g["v"], rows, g["score"],
                                      g["scale"], g["slope"])
        kind = g["kind"]
        F = out[0].size if out.shape[0] else 0
        H = lse.shape[1]
        res["out"] = stats(A.widen(g["gpu"]["out"][r0:r1]), out, kind, r0 * F)
        res["lse"] = stats(g["gpu"]["lse"][r0:r1], lse, "lse", r0 * H)
        if g["train"]:
            res["dq"] = stats(A.widen(g["gpu"]["dq"][r0:r1]), dq, kind, r0 * F)
    return res


def _cols_task(block):
    """Source columns [c0, c1): the oracle's dk, dv from every edge's (alpha, dS),
    compared with the GPU's rows of dk, dv."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    g = _G
    c0, c1 = block
    with threadpool_limits(1):
        dk, dv = A.column_pass(g["q"], g["dout"], g["ea"], g["ed"], g["order"], g["col_start"],
                               g["edge_row"], np.arange(c0, c1), g["scale"])
    F = dk[0].size if dk.shape[0] else 0
    return {"dk": stats(A.widen(g["gpu"]["dk"][c0:c1]), dk, g["kind"], c0 * F),
            "dv": stats(A.widen(g["gpu"]["dv"][c0:c1]), dv, g["kind"], c0 * F)}


def _run(pool, task, blocks):
    parts = {}
    for res in pool.imap_unordered(task, blocks):
        for k, v in res.items():
            parts.setdefault(k, []).append(v)
    return parts


def main(spec_path):
    import multiprocessing as mp

    spec = json.load(open(spec_path))
    os.environ["GRAPHGEN_CACHE"] = spec["graph_cache"]
    import graphgen as gg
    w = gg.WORKLOADS[spec["workload"]]
    n = spec.get("n")            # the workload's recipe at another node count (None: its own)
    t0 = time.perf_counter()
    ip, ix = gg.make_graph(w, n)
    feats = gg.make_features(w, n)
    train = bool(spec.get("train"))
    _G.update(ip=ip, ix=ix, q=feats[0], k=feats[1], v=feats[2], score=w.score,
              scale=spec["scale"], slope=spec.get("slope", 0.2), train=train,
              kind="bf16" if w.dtype == "bf16" else "f32",
              gpu={k: np.load(p, mmap_mode="r", allow_pickle=False)
                   for k, p in spec["gpu"].items()})
    if train:
        from oracle import attention as A
        _G["dout"] = gg.make_dout(w, n)
        E, H = ix.size, w.heads
        _G["ea"] = shared_array((E, H))
        _G["ed"] = shared_array((E, H))
        _G["order"], _G["col_start"], _G["edge_row"] = A.transpose_order(ip, ix)
    P = workers()
    prep = time.perf_counter() - t0
    t0 = time.perf_counter()
    ctx = mp.get_context("fork")
    with ctx.Pool(P) as pool:
        parts = _run(pool, _rows_task, balanced_blocks(ip, 8 * P))
        t_rows = time.perf_counter() - t0
        if train:
            colptr = _G["col_start"]
            parts.update(_run(pool, _cols_task, balanced_blocks(colptr, 8 * P)))
    total = time.perf_counter() - t0
    kinds = {"out": _G["kind"], "lse": "lse", "dq": _G["kind"], "dk": _G["kind"],
             "dv": _G["kind"]}
    result = {"workload": w.name, "nodes": int(ip.size - 1), "edges": int(ix.size),
              "workers": P, "prep_s": prep, "rows_s": t_rows, "total_s": total,
              "tensors": {k: merge(v, kinds[k]) for k, v in parts.items()}}
    result["ok"] = all(t["ok"] for t in result["tensors"].values())
    print(json.dumps(result), flush=True)
    return 0 if result["ok"] else 1


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
