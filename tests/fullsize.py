"""Every-element parity at full workload sizes, on the host: the fp64 oracle over every
row (and every source column) of a workload, in forked worker processes, compared element
by element with the results a GPU run saved to a directory.

Run as a child process, ``python -m tests.fullsize SPEC.json``, from a GPU test: the
workers are forked from this fresh process, which never touches the GPU.  SPEC names the
workload, the GRAPHGEN_CACHE directory holding its generated inputs, the saved GPU
results (.npy: bf16 as uint16 bit patterns) and the checks to run; the child prints one
JSON line with, per tensor, the parity verdict and its statistics.  The workload's score
picks the oracle: dot (forward, or with "train" the training step), gat and gatv2
(training steps: rows then source columns), max / min pooling (training step: out, arg
and slot exactly, then dx by feature columns).

Criteria (the same as tests/gpu_util.py, applied to every element):
  fp32 inputs:  |x - r| <= max(1e-5, 1e-4 |r|)
  bf16 inputs:  |x - r| <= 2e-2 max(|r|, rms(r)), rms over the whole tensor
  lse:          |x - r| <= max(1e-5, 1e-4 |r|), -inf exactly where r = -inf
  pooling out, arg, slot: exact (out as stored values, sign of zero included)
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


def stats_exact(got, ref, base=0, signed_zero=False):
    """Exact comparison of one block (floats by value, and by sign when signed_zero)."""
    got = np.asarray(got).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    bad = got != ref
    if signed_zero:
        bad |= np.signbit(got.astype(np.float64)) != np.signbit(ref.astype(np.float64))
    st = {"n": int(ref.size), "nonfinite": 0, "sum_r2": 0.0, "sum_e2": 0.0, "max_err": 0.0,
          "need_rms": 0.0, "n_bad": int(bad.sum()), "ninf_mismatch": 0, "worst": None}
    if bad.any():
        w = int(np.argmax(bad))
        st["worst"] = [base + w, float(got[w]), float(ref[w])]
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
    if kind == "exact":
        res["n_bad"] = sum(p["n_bad"] for p in parts)
        res["ok"] = res["n_bad"] == 0
    elif kind == "bf16":
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
    kind, gpu, score = g["kind"], g["gpu"], g["score"]
    with threadpool_limits(1):
        if score in ("max", "min"):
            return _pool_rows_task(block)
        grads = {}
        if not g["train"]:
            out, lse = A.forward_rows(ip, ix, g["q"], g["k"], g["v"], rows, score, g["scale"],
                                      g["slope"])
        elif score == "dot":
            out, lse, grads["dq"], ea, ed = A.row_pass(ip, ix, g["q"], g["k"], g["v"],
                                                       g["dout"], rows, g["scale"])
        elif score == "gat":
            out, lse, grads["ds"], ea, ed = A.row_pass_gat(ip, ix, g["q"], g["k"], g["v"],
                                                           g["dout"], rows, g["scale"],
                                                           g["slope"])
        else:  # gatv2: q, k, v = xd, xs, attn
            out, lse, grads["dxd"], ea, ed, da = A.row_pass_gatv2(
                ip, ix, g["q"], g["k"], g["v"], g["dout"], rows, g["scale"], g["slope"])
            res["dattn_part"] = da.tolist()
        if g["train"]:
            g["ea"][ip[r0]:ip[r1]] = ea
            g["ed"][ip[r0]:ip[r1]] = ed
        F = out[0].size if out.shape[0] else 0
        H = lse.shape[1]
        res["out"] = stats(A.widen(gpu["out"][r0:r1]), out, kind, r0 * F)
        res["lse"] = stats(gpu["lse"][r0:r1], lse, "lse", r0 * H)
        for name, ref in grads.items():
            per = ref[0].size if ref.shape[0] else 0
            res[name] = stats(A.widen(gpu[name][r0:r1]), ref, kind, r0 * per)
    return res


def _pool_rows_task(block):
    """Rows [r0, r1) of min / max pooling: out, arg and slot exactly; the arg goes to the
    shared array for the backward."""
    from oracle import attention as A
    from oracle import reduction as R
    g = _G
    r0, r1 = block
    rows = np.arange(r0, r1)
    out, arg = R.reduce_rows(g["ip"], g["ix"], g["q"], rows, g["score"])
    g["arg"][r0:r1] = arg
    F = out.shape[1]
    # slots index the rows of the plan the GPU ran (its exported indices)
    slot = R.slots_of(g["ip"], g["plan_ix"], rows, arg)
    gslot = np.asarray(g["gpu"]["slot"][r0:r1]).reshape(len(rows), F).astype(np.int64)
    gslot[gslot == g["slot_none"]] = -1
    return {"out": stats_exact(A.widen(g["gpu"]["out"][r0:r1]).reshape(len(rows), F), out,
                               r0 * F, signed_zero=True),
            "arg": stats_exact(np.asarray(g["gpu"]["arg"][r0:r1]).reshape(len(rows), F), arg,
                               r0 * F),
            "slot": stats_exact(gslot, slot, r0 * F)}


def _pool_dx_task(fs):
    """Feature columns [f0, f1) of the pooling backward: the scatter-form oracle from the
    oracle's own arg, compared with the GPU's dx."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    from oracle import reduction as R
    g = _G
    f0, f1 = fs
    N = g["ip"].size - 1
    with threadpool_limits(1):
        dx = R.reduce_backward(g["arg"][:, f0:f1], g["dout_flat"][:, f0:f1], N)
    got = A.widen(np.asarray(g["gpu"]["dx"]).reshape(N, -1)[:, f0:f1])
    st = stats(got, dx, g["kind"])
    st["worst"] = None if st["worst"] is None else \
        [int(st["worst"][0] // (f1 - f0)) * g["F"] + f0 + st["worst"][0] % (f1 - f0)] + \
        st["worst"][1:]
    return {"dx": st}


def _cols_task(block):
    """Source columns [c0, c1): the oracle's dk, dv from every edge's (alpha, dS),
    compared with the GPU's rows of dk, dv."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    g = _G
    c0, c1 = block
    cols = np.arange(c0, c1)
    tr = (g["ea"], g["ed"], g["order"], g["col_start"], g["edge_row"], cols)
    with threadpool_limits(1):
        if g["score"] == "dot":
            ref = dict(zip(("dk", "dv"), A.column_pass(g["q"], g["dout"], *tr, g["scale"])))
        elif g["score"] == "gat":
            ref = dict(zip(("dt", "dv"), A.column_pass_gat(g["q"], g["k"], g["dout"], *tr,
                                                           g["scale"], g["slope"])))
        else:
            ref = {"dxs": A.column_pass_gatv2(g["q"], g["k"], g["v"], g["dout"], *tr,
                                              g["scale"], g["slope"])}
    res = {}
    for name, r in ref.items():
        per = r[0].size if r.shape[0] else 0
        res[name] = stats(A.widen(g["gpu"][name][c0:c1]), r, g["kind"], c0 * per)
    return res


def _run(pool, task, blocks):
    parts = {}
    for res in pool.imap_unordered(task, blocks):
        for k, v in res.items():
            parts.setdefault(k, []).append(v)
    return parts


def _feature_blocks(F, k):
    cuts = np.unique(np.linspace(0, F, min(F, k) + 1).astype(np.int64))
    return [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:])]


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
    pool_mode = w.score in ("max", "min")
    _G.update(ip=ip, ix=ix, q=feats[0], k=None if pool_mode else feats[1],
              v=None if pool_mode else feats[2], score=w.score, scale=spec.get("scale"),
              slope=spec.get("slope", 0.2), train=train,
              kind="bf16" if w.dtype == "bf16" else "f32",
              gpu={k: np.load(p, mmap_mode="r", allow_pickle=False)
                   for k, p in spec["gpu"].items()})
    if pool_mode:
        from oracle import attention as A
        N, F = ip.size - 1, w.heads * w.dim
        _G["plan_ix"] = np.load(spec["plan_indices"], allow_pickle=False)
        _G["slot_none"] = (1 << (8 * _G["gpu"]["slot"].dtype.itemsize)) - 1
        _G["arg"] = shared_array((N, F), np.int64)
        _G["F"] = F
        _G["dout_flat"] = gg.make_dout(w, n).reshape(N, F)
    elif train:
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
        if pool_mode and train:
            parts.update(_run(pool, _pool_dx_task, _feature_blocks(_G["F"], 4 * P)))
        elif train:
            colptr = _G["col_start"]
            parts.update(_run(pool, _cols_task, balanced_blocks(colptr, 8 * P)))
    total = time.perf_counter() - t0
    kinds = {"lse": "lse", "out": "exact" if pool_mode else _G["kind"], "arg": "exact",
             "slot": "exact"}
    da_parts = parts.pop("dattn_part", None)
    tensors = {k: merge(v, kinds.get(k, _G["kind"])) for k, v in parts.items()}
    if da_parts is not None:  # GATv2: the attention-vector gradient, summed over all rows
        from oracle import attention as A
        da = np.sum(np.asarray(da_parts, np.float64), axis=0)
        tensors["dattn"] = merge([stats(np.asarray(_G["gpu"]["dattn"], np.float64), da,
                                        _G["kind"])], _G["kind"])
    result = {"workload": w.name, "nodes": int(ip.size - 1), "edges": int(ix.size),
              "workers": P, "prep_s": prep, "rows_s": t_rows, "total_s": total,
              "tensors": tensors}
    result["ok"] = all(t["ok"] for t in result["tensors"].values())
    print(json.dumps(result), flush=True)
    return 0 if result["ok"] else 1


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
