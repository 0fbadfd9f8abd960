"""Benchmark of the fused CSR graph-attention layer on one MI355X.

A step is one training step of the layer on the 1M-node Chung-Lu workload (gamma 2.1,
average in-degree 50 plus self-loops, H = 8, d = 32, bf16 with fp32 accumulation): the
forward (scores -> online softmax -> weighted V, saving the per-row log-sum-exp), then
the backward (dQ over CSR, dK/dV over the cached transpose).  The graph plan is built
once per graph, before the timed region, as the method caches graph metadata.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
    python bench.py --ingest-counters DIR --workload NAME   # rocprofv3 CSV -> profiles/

Prints one JSON line.  ``value`` is edges/s of the whole step (E / step time) with
inputs resident in HBM.  ``roofline`` rates the dominant kernel against the 8 TB/s HBM
peak by the L2-miss bytes its launches move (rocprofv3 FETCH_SIZE and WRITE_SIZE, from
the committed counter runs of the same kernel sources and plan) over its average
duration measured here with HIP events on the launch stream: an upper bound on its HBM
rate, as the 256 MB MALL may serve some of those misses; ``compulsory`` beside it is the
lower bound (every operand and output row once).  ``floors`` time gather-only probes
over the same plan's work lists; ``gather_ceiling`` gathers random rows from tables of
growing size.  ``cpu_baseline`` is the fp64 oracle timed on this host on a time-boxed
uniform sample of rows (same edges/s unit).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import graphgen as gg  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# oracle worker processes: every CPU this process may run on, at most the 16 host CPUs
# allotted to each GPU
HOST_CPUS_PER_GPU = 16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# XCD split thresholds of the attention workloads' plans (rows, transpose columns): a sweep
# on the 1M-node training step gave 19.19 ms unsplit, 17.54 ms at 256 / 1024, 17.71 ms at
# 512 / 512 and 18.31 ms at 128 / 128 (chunk partials outgrow the L2 gain below ~256)
XCD_SPLIT_ROWS, XCD_SPLIT_COLS = 256, 1024
# the min / max reduction's chunk partials (value, id, edge) are larger, so its merge is
# dearer: 7.85 ms unsplit, 7.56 ms at 256 / 1024, 7.40 ms at 512 / 512 on the 1M max step
XCD_SPLIT_REDUCE = 512
# column chunk of the dot-score workloads' split plans: a sweep on the 1M training step
# (columns split above 1024) gave 17.57 ms at the automatic 512-edge chunk, 17.52-17.53 ms
# at 1024 (and 537 instead of 556 MB of backward workspace), 17.56 ms at 2048, 17.55 at 4096
XCD_SPLIT_COL_CHUNK = 1024


# ---------------------------------------------------------------- algorithmic bytes

def algorithmic_bytes(kernel, N, E, H, d, b, score="dot"):
    """Logical bytes of a launch: the CSR (or transpose) once, one read of each gathered
    row per edge, each per-node operand once and each output once.  Power-law graphs
    re-gather hot rows, which the L2 and the MALL serve, so these bytes over the time can
    exceed the HBM peak: a work rate, not a fraction of any memory roofline."""
    F = H * d
    csr = 4 * (N + 1) + 4 * E
    if kernel == "fwd_main":
        if score == "gat":      # V_j + t_j per edge; s, out, lse per node
            return csr + E * (F * b + 4 * H) + 4 * N * H + N * F * b + 4 * N * H
        if score == "gatv2":    # xs_j per edge (score operand and message); xd, out, lse; attn
            return csr + E * F * b + 2 * N * F * b + 4 * N * H + 4 * F
        return csr + 2 * E * F * b + 2 * N * F * b + 4 * N * H   # K_j + V_j; Q, out, lse
    if kernel == "bwd_dq_main":    # K_j + V_j per edge; Q, dOut, lse; dQ, (lse, D) record
        return csr + 2 * E * F * b + 2 * N * F * b + 4 * N * H + N * F * b + 8 * N * H
    if kernel == "bwd_dkdv_main":  # Q_i + dOut_i + record_i per edge; K, V; dK, dV
        return csr + E * (2 * F * b + 8 * H) + 2 * N * F * b + 2 * N * F * b
    if kernel == "bwd_gat_rows_main":    # t_j + V_j per edge; s, dOut, lse; ds, record
        return csr + E * (4 * H + F * b) + 4 * N * H + N * F * b + 4 * N * H + 4 * N * H \
            + 8 * N * H
    if kernel == "bwd_gat_cols_main":    # s_i + dOut_i + record_i per edge; t, V; dt, dV
        return csr + E * (4 * H + F * b + 8 * H) + 4 * N * H + N * F * b + 4 * N * H + N * F * b
    if kernel == "bwd_gatv2_rows_main":  # xs_j per edge; xd, dOut, lse; dxd, record; attn
        return csr + E * F * b + 2 * N * F * b + 4 * N * H + N * F * b + 8 * N * H + 4 * F
    if kernel == "bwd_gatv2_cols_main":  # xd_i + dOut_i + record_i per edge; xs; dxs; attn
        return csr + E * (2 * F * b + 8 * H) + N * F * b + N * F * b + 4 * F
    if kernel == "reduce_fwd_main":      # x_j per edge; out, int32 arg and 16-bit slot
        return csr + E * F * b + N * F * b + 4 * N * F + 2 * N * F
    if kernel == "reduce_bwd_main":      # per transpose edge its row position and the row's
        # 16-bit slots; each dout element once (it matches once); dx
        return csr + 4 * E + 2 * E * F + N * F * b + N * F * b
    return None


REDUCTIONS = ("max", "min")


def step_bytes(N, E, H, d, b, backward, score="dot"):
    if score in REDUCTIONS:
        tot = algorithmic_bytes("reduce_fwd_main", N, E, H, d, b, score)
        if backward:
            tot += algorithmic_bytes("reduce_bwd_main", N, E, H, d, b, score)
        return tot
    tot = algorithmic_bytes("fwd_main", N, E, H, d, b, score)
    if backward and score == "gatv2":
        tot += algorithmic_bytes("bwd_gatv2_rows_main", N, E, H, d, b, score)
        tot += algorithmic_bytes("bwd_gatv2_cols_main", N, E, H, d, b, score)
    elif backward and score == "gat":
        tot += algorithmic_bytes("bwd_gat_rows_main", N, E, H, d, b, score)
        tot += algorithmic_bytes("bwd_gat_cols_main", N, E, H, d, b, score)
    elif backward:
        tot += algorithmic_bytes("bwd_dq_main", N, E, H, d, b, score)
        tot += algorithmic_bytes("bwd_dkdv_main", N, E, H, d, b, score)
    return tot


def compulsory_bytes(kernel, N, E, H, d, b, score="dot"):
    """Bytes a launch cannot avoid moving from HBM: the CSR (or transpose) once and every
    operand and output row once, however often the pass gathers it.  Over the launch's
    time, a lower bound on its HBM rate."""
    F = H * d
    row = N * F * b               # one [N, H, d] operand
    nh = 4 * N * H                # one fp32 [N, H] array
    csr = 4 * (N + 1) + 4 * E
    if kernel == "fwd_main":
        if score == "gat":      # s, t, V; out, lse
            return csr + 2 * nh + row + row + nh
        if score == "gatv2":    # xd, xs; out, lse; attn
            return csr + 2 * row + row + nh + 4 * F
        return csr + 3 * row + row + nh                       # Q, K, V; out, lse
    if kernel == "bwd_dq_main":    # Q, K, V, dOut, lse; dQ, record
        return csr + 4 * row + nh + row + 2 * nh
    if kernel == "bwd_dkdv_main":  # Q, dOut, record, K, V; dK, dV
        return csr + 4 * row + 2 * nh + 2 * row
    if kernel == "bwd_gat_rows_main":    # s, t, V, dOut, lse; ds, record
        return csr + 2 * nh + 2 * row + nh + nh + 2 * nh
    if kernel == "bwd_gat_cols_main":    # s, dOut, record, t, V; dt, dV
        return csr + nh + row + 2 * nh + nh + row + nh + row
    if kernel == "bwd_gatv2_rows_main":  # xs, xd, dOut, lse, attn; dxd, record
        return csr + 3 * row + nh + 4 * F + row + 2 * nh
    if kernel == "bwd_gatv2_cols_main":  # xd, dOut, record, xs, attn; dxs
        return csr + 3 * row + 2 * nh + 4 * F + row
    if kernel == "reduce_fwd_main":      # x; out, int32 arg, 16-bit slot
        return csr + row + row + 4 * N * F + 2 * N * F
    if kernel == "reduce_bwd_main":      # csc_rel, slots, dOut; dx
        return csr + 4 * E + 2 * N * F + row + row
    return None


# ---------------------------------------------------------------- CPU baseline (oracle)

_SHARED = {}


def _cpu_worker(args):
    rows, deadline_s, backward = args
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    g = _SHARED
    t0 = time.perf_counter()
    done_rows = done_edges = 0
    with threadpool_limits(1):
        for s in range(0, rows.size, 128):
            batch = rows[s:s + 128]
            if g["score"] == "gatv2":
                if backward:
                    A.train_step_rows_gatv2(g["ip"], g["ix"], g["q"], g["k"], g["v"], g["dout"],
                                            batch, g["scale"], g["slope"])
                else:
                    A.forward_gatv2_rows(g["ip"], g["ix"], g["q"], g["k"], g["v"], batch,
                                         g["scale"], g["slope"])
            elif g["score"] in REDUCTIONS:
                from oracle import reduction as R
                if backward:
                    R.train_step_rows(g["ip"], g["ix"], g["q"], g["dout"], batch, g["score"])
                else:
                    R.reduce_rows(g["ip"], g["ix"], g["q"], batch, g["score"])
            elif backward and g["score"] == "gat":
                A.train_step_rows_gat(g["ip"], g["ix"], g["q"], g["k"], g["v"], g["dout"],
                                      batch, g["scale"], g["slope"])
            elif backward:
                A.train_step_rows(g["ip"], g["ix"], g["q"], g["k"], g["v"], g["dout"], batch,
                                  g["scale"])
            else:
                A.forward_rows(g["ip"], g["ix"], g["q"], g["k"], g["v"], batch, g["score"],
                               g["scale"], g["slope"])
            done_rows += batch.size
            done_edges += int((g["ip"][batch + 1] - g["ip"][batch]).sum())
            if time.perf_counter() - t0 > deadline_s:
                break
    return done_rows, done_edges, time.perf_counter() - t0


def cpu_baseline(ip, ix, feats, dout, w, scale, budget_s):
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    cores = min(HOST_CPUS_PER_GPU, affinity)
    red = w.score in REDUCTIONS
    _SHARED.update(ip=ip, ix=ix, q=feats[0], k=None if red else feats[1],
                   v=None if red else feats[2], dout=dout, scale=scale, score=w.score, slope=0.2)
    rng = np.random.default_rng(12345)
    n = ip.size - 1
    # a bounded row sample; the reduction oracle is fast enough to take every row
    rows = rng.permutation(n)[: n if red else min(n, 400_000)]
    parts = np.array_split(rows, cores)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        res = pool.map(_cpu_worker, [(p, budget_s, w.backward) for p in parts])
    wall = time.perf_counter() - t0
    r = sum(x[0] for x in res)
    e = sum(x[1] for x in res)
    longest = max(x[2] for x in res)
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    what = "forward+backward" if w.backward else "forward"
    if red:
        what = f"{w.score}-pooling {what} (backward: the rows' routed gradient)"
    return {
        "value": e / longest, "unit": "edges/s", "cores": cores, "affinity_cpus": affinity,
        "kind": "oracle",
        "sample": f"{what} of {r} uniformly sampled rows ({e} edges) of the same graph, "
                  f"time-boxed to {budget_s:.0f} s per worker on {cores} fork workers "
                  f"(fp64 numpy per-row oracle, 1 BLAS thread each); wall {wall:.1f} s; "
                  f"cpu: {cpu}",
    }


def relabel(ip, ix, feats, dout, old_of_new):
    """The same graph with node old_of_new[k] renamed k; per-node arrays move with their
    nodes (per-graph arrays such as the GATv2 attention vector stay)."""
    n = ip.size - 1
    new_of_old = np.empty(n, np.int64)
    new_of_old[old_of_new] = np.arange(n)
    dst = new_of_old[np.repeat(np.arange(n), np.diff(ip))]
    src = new_of_old[ix]
    ip2, ix2 = gg.csr_from_edges(n, src, dst)
    feats = tuple(np.ascontiguousarray(f[old_of_new]) if f.shape[0] == n else f for f in feats)
    dout = None if dout is None else np.ascontiguousarray(dout[old_of_new])
    return ip2, ix2, feats, dout


def order_by_out_degree(ip, ix):
    """Node order ablation: rank by out-degree (descending, ties by old id), so the hot
    source rows are contiguous."""
    n = ip.size - 1
    odeg = np.bincount(ix, minlength=n)
    return np.lexsort((np.arange(n), -odeg))


def order_rcm(ip, ix):
    """Node order ablation: reverse Cuthill-McKee on the symmetrised pattern (scipy), a
    bandwidth-reducing locality order: neighbours get nearby ids."""
    import scipy.sparse as sp
    from scipy.sparse.csgraph import reverse_cuthill_mckee
    n = ip.size - 1
    a = sp.csr_matrix((np.ones(ix.size, np.int8), ix, ip), shape=(n, n))
    sym = (a + a.T).tocsr()
    sym.sum_duplicates()
    return np.asarray(reverse_cuthill_mckee(sym, symmetric_mode=True), dtype=np.int64)


# ---------------------------------------------------------------- GPU

def capi_ws(fn, plan, features):
    from ctypes import byref, c_size_t
    from sparse_graph_attention_02_amd import capi
    v = c_size_t()
    getattr(capi, fn)(plan.handle, features, byref(v))
    return v.value


def to_dev(x):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def xcd_split_of(w, rows=None, cols=None):
    """(row, column) XCD split thresholds of the plan for workload w: the given values, else
    the defaults (attention: rows 256 / columns 1024; min / max reduction: 512 / 512). A
    column threshold left open follows the rows: 0 when they are 0, else at least the
    column default and at least the row threshold."""
    reduction = w.score in ("max", "min")
    if rows is None:
        rows = XCD_SPLIT_REDUCE if reduction else XCD_SPLIT_ROWS
    if cols is None:
        col_default = XCD_SPLIT_REDUCE if reduction else XCD_SPLIT_COLS
        cols = 0 if rows == 0 else max(col_default, rows)
    return rows, cols


# the device source file of each kernel family; every kernel also includes the shared
# device and internal headers
KERNEL_SOURCES = (("fwd_", "fwd.hip"), ("bwd_dq_", "bwd.hip"), ("bwd_dkdv_", "bwd.hip"),
                  ("bwd_gat_", "bwd_gat.hip"), ("bwd_gatv2_", "bwd_gatv2.hip"),
                  ("reduce_", "reduce.hip"), ("gather_probe", "probe.hip"),
                  ("copy_probe", "probe.hip"))
SHARED_HEADERS = ("ga_device.h", "ga_internal.h")


def kernel_source(kernel):
    """The .hip file that defines `kernel` (None if unknown)."""
    for prefix, src in KERNEL_SOURCES:
        if kernel.startswith(prefix):
            return src
    return None


def bench_plan_kw(w, rows=None, cols=None, col_chunk=None):
    """The XCD-split plan options bench.py runs workload w with (rows / columns split
    thresholds as in xcd_split_of; the dot-score workloads' split transpose also takes
    1024-edge column chunks unless a chunk is given)."""
    rows, cols = xcd_split_of(w, rows, cols)
    kw = dict(xcd_split_min_deg_exclusive=rows, col_xcd_split_min_deg_exclusive=cols)
    if col_chunk is None and cols > 0 and w.score == "dot":
        col_chunk = XCD_SPLIT_COL_CHUNK
    if col_chunk is not None:
        kw["col_hub_chunk"] = col_chunk
    return kw


def source_digest(kernel=None):
    """Digest of the device sources a kernel is built from (its .hip file and the shared
    headers; every device source when `kernel` is None or unknown): counters taken on
    other sources do not describe that kernel."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_graph_attention_02_amd", "csrc")
    src = kernel_source(kernel) if kernel else None
    files = sorted(os.listdir(csrc)) if src is None else sorted((src,) + SHARED_HEADERS)
    for f in files:
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


# what fixes the work a kernel launch does besides its sources: the plan (bins, chunks,
# schedules, slices) and the node order
PLAN_KEYS = ("light_max_deg", "hub_min_deg_exclusive", "hub_chunk", "n_row_light",
             "n_row_medium", "n_row_hub", "n_row_chunks", "n_col_hub", "n_col_chunks",
             "max_in_degree", "max_out_degree", "rows_sorted", "feature_slices",
             "col_hub_min_deg_exclusive", "col_hub_chunk", "xcd_split_min_deg_exclusive",
             "col_xcd_split_min_deg_exclusive", "n_row_sched", "n_col_sched")


def measured_traffic(workload, kernel, plan, node_order, path=None):
    """L2-miss bytes per launch of `kernel` from the committed rocprofv3 counter runs, if
    they were taken on the current kernel sources, the same plan and node order (else
    None)."""
    try:
        t = json.load(open(path or TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = t.get(workload, {}).get(kernel)
    if not rec or rec.get("source_digest") != source_digest(kernel):
        return None
    if rec.get("plan") != {k: plan[k] for k in PLAN_KEYS} or \
            rec.get("node_order", "as-generated") != node_order:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------- counter ingestion

def _kernel_short(name):
    """`void ga::(anonymous namespace)::fwd_main<unsigned short, 32, 4, 0, 8>(ga::FwdArgs)`
    -> `fwd_main<unsigned short, 32, 4, 0, 8>`."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("ga::(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def _kernel_base(n):
    return n.split("<")[0]


def _last_json_line(path):
    last = None
    for line in open(path):
        if line.startswith("{"):
            last = line
    if last is None:
        raise ValueError(f"{path}: no bench line")
    return json.loads(last)


def ingest_counters(run_dir, workload, profiles_dir=None, traffic_path=None):
    """Summarise one workload's rocprofv3 runs of this script into profiles/.

    run_dir holds `kt.log` (the output of the kernel-trace run, whose last line is its
    bench line), `kt/**/*kernel_stats.csv` (rocprofv3 --kernel-trace --stats), and one
    folder per counter pass `p<k>/**/*counter_collection.csv` with `p<k>.counters` naming
    its counters.  Writes <workload>.kernel_trace.txt and <workload>.counters.txt and the
    workload's records in traffic.json: per kernel, L2-miss bytes per launch =
    FETCH_SIZE * 1024 * f + WRITE_SIZE * 1024 * w, where f and w make the library's copy
    kernel, which reads and writes exactly 1 GiB per launch in every bench run, read 1 GiB
    each; with the counters' source digest, plan and node order.  Returns the records."""
    import csv
    import glob
    from collections import defaultdict
    prof = profiles_dir or os.path.join(ROOT, "profiles")
    tpath = traffic_path or os.path.join(prof, "traffic.json")
    bl = _last_json_line(os.path.join(run_dir, "kt.log"))
    cfg = bl["config"]
    if cfg["workload"] != workload:
        raise ValueError(f"{run_dir}: bench line of {cfg['workload']}, not {workload}")
    N, E, H, dim = cfg["nodes"], cfg["edges"], cfg["heads"], cfg["dim"]
    desc = f"{workload} (N={N}, E={E}, H={H}, d={dim}, {bl['dtype']}, {cfg['step']})"
    plan = cfg["plan"]
    split = (f"xcd split rows {plan.get('xcd_split_min_deg_exclusive', 0)} / columns "
             f"{plan.get('col_xcd_split_min_deg_exclusive', 0)}; node order "
             f"{cfg.get('node_order', 'as-generated')}")
    stats = glob.glob(os.path.join(run_dir, "kt", "**", "*kernel_stats.csv"), recursive=True)
    if len(stats) != 1:
        raise ValueError(f"{run_dir}/kt: expected one kernel_stats.csv, found {len(stats)}")
    st = [(_kernel_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e6,
           float(r["MinNs"]) / 1e6, float(r["MaxNs"]) / 1e6, float(r["Percentage"]))
          for r in csv.DictReader(open(stats[0]))]
    lib = {k: v["avg_ms"] for k, v in bl["kernels"].items()}
    cmd_kt = ("rocprofv3 --kernel-trace --stats --output-format csv -d <run>/kt -o kt -- "
              f"python3 bench.py --cpu-budget 0 --ceiling-gathers 0 --workload {workload}")
    if cfg.get("node_order", "as-generated") != "as-generated":
        cmd_kt += f" --order {cfg['node_order']}"
    out = [f"# rocprofv3 kernel trace: {desc}",
           f"# command (repo root): {cmd_kt} > <run>/kt.log",
           f"# plan: {split}",
           f"# bench line of the same run: ms_per_step={bl['ms_per_step']:.3f}  "
           f"value={bl['value']:.4g} edges/s",
           "# library event timers of the same run (avg ms): "
           + ", ".join(f"{k}={v:.4f}" for k, v in lib.items()),
           f"# written by: python3 bench.py --ingest-counters <run> --workload {workload}",
           "", f"{'kernel':52s} {'calls':>6s} {'avg_ms':>9s} {'min_ms':>9s} {'max_ms':>9s} "
           f"{'pct':>6s}"]
    st = [x for x in st if kernel_source(_kernel_base(x[0]))]   # the library's kernels
    for n, c, a, mn, mx, pc in st:
        out.append(f"{n:52s} {c:6d} {a:9.4f} {mn:9.4f} {mx:9.4f} {pc:6.2f}")
    os.makedirs(prof, exist_ok=True)
    open(os.path.join(prof, f"{workload}.kernel_trace.txt"), "w").write("\n".join(out) + "\n")
    avg = {_kernel_base(n): a for n, c, a, mn, mx, pc in st}
    # counters: kernel -> counter -> mean over its dispatches
    vals = defaultdict(lambda: defaultdict(list))
    passes = []
    for cf in sorted(glob.glob(os.path.join(run_dir, "p*.counters"))):
        pname = os.path.basename(cf)[:-len(".counters")]
        passes.append(open(cf).read().strip())
        for f in glob.glob(os.path.join(run_dir, pname, "**", "*counter_collection.csv"),
                           recursive=True):
            for r in csv.DictReader(open(f)):
                vals[_kernel_short(r["Kernel_Name"])][r["Counter_Name"]].append(
                    float(r["Counter_Value"]))
    cnt = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    cp = next((c for k, c in cnt.items() if _kernel_base(k) == "copy_probe"), None)
    if not cp or "FETCH_SIZE" not in cp or "WRITE_SIZE" not in cp:
        raise ValueError(f"{run_dir}: no FETCH_SIZE / WRITE_SIZE of copy_probe to calibrate")
    ff = (1 << 30) / (cp["FETCH_SIZE"] * 1024)
    wf = (1 << 30) / (cp["WRITE_SIZE"] * 1024)
    order_arg = "" if cfg.get("node_order", "as-generated") == "as-generated" \
        else f" --order {cfg['node_order']}"
    o = [f"# rocprofv3 counters: {desc}", f"# plan: {split}",
         "# one run per pass (repo root):"]
    o += [f"#   timeout -s KILL 240 rocprofv3 --pmc {p} --output-format csv -d <run>/p{k + 1} "
          f"-o p{k + 1} -- python3 bench.py --cpu-budget 0 --ceiling-gathers 0 --workload "
          f"{workload}{order_arg} --steps 1 --warmup 1" for k, p in enumerate(passes)]
    o += [f"# written by: python3 bench.py --ingest-counters <run> --workload {workload}",
          "#", "# calibration with the library copy kernel (1 GiB read + 1 GiB written per "
          "launch, in every run):",
          f"#   FETCH_SIZE reads {cp['FETCH_SIZE']:.0f} KiB -> fetch factor {ff:.4f};  "
          f"WRITE_SIZE reads {cp['WRITE_SIZE']:.0f} KiB -> write factor {wf:.4f}",
          "# traffic = FETCH_SIZE*1024*fetch_factor + WRITE_SIZE*1024*write_factor, bytes per "
          "launch: L2 misses (TCC to EA requests), which the 256 MB MALL in front of HBM may "
          "serve, so an upper bound on HBM bytes; compulsory = every operand and output row "
          "once, a lower bound.", ""]
    b = 2 if bl["dtype"] == "bf16" else 4
    score = cfg["score"]
    recs = {}
    for k in sorted(cnt):
        c = cnt[k]
        kb = _kernel_base(k)
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c or not kernel_source(kb):
            continue
        fb, wb = c["FETCH_SIZE"] * 1024 * ff, c["WRITE_SIZE"] * 1024 * wf
        t = fb + wb
        line = f"   fetch {fb / 1e9:9.3f} GB   write {wb / 1e9:8.3f} GB   traffic " \
               f"{t / 1e9:9.3f} GB/launch"
        logical = algorithmic_bytes(kb, N, E, H, dim, b, score)
        comp = compulsory_bytes(kb, N, E, H, dim, b, score)
        if logical:
            line += f"   logical {logical / 1e9:9.3f} GB  compulsory {comp / 1e9:7.3f} GB  " \
                    f"traffic/logical {t / logical:.3f}"
        o += [k, line]
        a = avg.get(kb)
        if a:
            l2 = f"   avg {a:.4f} ms -> traffic rate {t / (a * 1e-3) / 1e9:8.1f} GB/s " \
                 f"({t / (a * 1e-3) / 1e9 / HBM_PEAK_GBPS:.3f} of 8 TB/s)"
            if logical:
                l2 += f", compulsory rate {comp / (a * 1e-3) / 1e9:7.1f} GB/s, logical rate " \
                      f"{logical / (a * 1e-3) / 1e9:8.1f} GB/s"
            o.append(l2)
        hr = None
        if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
            hr = c["TCC_HIT_sum"] / max(1.0, c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
            extra = ""
            if "TCC_EA0_RDREQ_sum" in c:
                extra = f"   EA read requests {c['TCC_EA0_RDREQ_sum']:.4g}"
                if "TCC_EA0_RDREQ_128B_sum" in c:
                    extra += f" (128B {c['TCC_EA0_RDREQ_128B_sum']:.4g})"
            o.append(f"{extra}   L2 hit {c['TCC_HIT_sum']:.4g} miss {c['TCC_MISS_sum']:.4g} -> "
                     f"hit rate {hr:.3f}")
        sq = [x for x in ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS",
                          "SQ_INSTS_SALU", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES",
                          "SQ_ACTIVE_INST_VALU") if x in c]
        if sq:
            o.append("   SQ: " + "  ".join(f"{x[3:].lower()} {c[x]:.4g}" for x in sq))
            if "SQ_INSTS_VALU" in c and logical and E:
                o.append(f"   VALU wave-instructions per edge {c['SQ_INSTS_VALU'] / E:.2f}")
        o.append("")
        if kb != "copy_probe":
            recs[kb] = {"bytes_per_launch": t, "fetch_bytes": fb, "write_bytes": wb,
                        "fetch_factor": ff, "write_factor": wf, "l2_hit_rate": hr,
                        "source_digest": source_digest(kb),
                        "plan": {q: plan[q] for q in PLAN_KEYS},
                        "node_order": cfg.get("node_order", "as-generated")}
    open(os.path.join(prof, f"{workload}.counters.txt"), "w").write("\n".join(o))
    try:
        tj = json.load(open(tpath))
    except (OSError, ValueError):
        tj = {}
    tj[workload] = recs
    with open(tpath, "w") as f:
        json.dump(tj, f, indent=1, sort_keys=True)
    return recs


# ---------------------------------------------------------------- main

def _rates(bytes_, ms):
    return None if bytes_ is None or not ms else bytes_ / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="chunglu1m_train_bf16", choices=sorted(gg.WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds per worker for the oracle baseline (0 = skip)")
    ap.add_argument("--light", type=int, default=None)
    ap.add_argument("--hub", type=int, default=None)
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--col-hub", type=int, default=None)
    ap.add_argument("--col-chunk", type=int, default=None)
    ap.add_argument("--xcd-split", type=int, default=None,
                    help="rows longer than this are regrouped by source id mod 8 and their "
                         "chunks scheduled to the matching XCD (0 = off; default %d for the "
                         "attention workloads, %d for the reductions)"
                         % (XCD_SPLIT_ROWS, XCD_SPLIT_REDUCE))
    ap.add_argument("--col-xcd-split", type=int, default=None,
                    help="the same for transpose columns (default %d for the attention "
                         "workloads, %d for the reductions)" % (XCD_SPLIT_COLS, XCD_SPLIT_REDUCE))
    ap.add_argument("--slices", type=int, default=None,
                    help="feature slices per XCD group (0 = automatic, 1 = off, 2, 4, 8)")
    ap.add_argument("--order", choices=["as-generated", "out-degree", "rcm"],
                    default="as-generated",
                    help="node order ablation: relabel nodes by descending out-degree (hot "
                         "source rows contiguous) or by reverse Cuthill-McKee (locality) "
                         "before the run")
    ap.add_argument("--ceiling-gathers", type=int, default=1 << 25,
                    help="rows gathered per table size by the random-table ceiling (0 = skip)")
    ap.add_argument("--ingest-counters", metavar="DIR", default=None,
                    help="summarise the rocprofv3 runs in DIR for --workload into profiles/ "
                         "(no GPU)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the fused layer is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.ingest_counters:
        recs = ingest_counters(args.ingest_counters, args.workload)
        print(json.dumps({k: round(v["bytes_per_launch"] / 1e9, 3) for k, v in recs.items()}))
        return

    w = gg.WORKLOADS[args.workload]
    pkw = bench_plan_kw(w, args.xcd_split, args.col_xcd_split, args.col_chunk)
    args.xcd_split = pkw["xcd_split_min_deg_exclusive"]
    args.col_xcd_split = pkw["col_xcd_split_min_deg_exclusive"]
    args.col_chunk = pkw.get("col_hub_chunk")
    t0 = time.perf_counter()
    ip, ix = gg.make_graph(w)
    feats = gg.make_features(w)
    dout = gg.make_dout(w) if w.backward else None
    if args.order != "as-generated":
        order = order_by_out_degree(ip, ix) if args.order == "out-degree" else order_rcm(ip, ix)
        ip, ix, feats, dout = relabel(ip, ix, feats, dout, order)
    gen_s = time.perf_counter() - t0
    N, E, H, d = ip.size - 1, ix.size, w.heads, w.dim
    b = 2 if w.dtype == "bf16" else 4
    scale = float(np.float32(1 / math.sqrt(d))) if w.score == "dot" else 1.0
    print(f"[bench] {w.name}: N={N} E={E} H={H} d={d} {w.dtype} {w.score} "
          f"backward={w.backward} (inputs {gen_s:.1f}s)", file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(ip, ix, feats, dout, w, scale, args.cpu_budget)
        print(f"[bench] cpu oracle: {cpu['value']:.3g} edges/s on {cpu['cores']} cores "
              f"(affinity {cpu['affinity_cpus']})", file=sys.stderr, flush=True)

    # ---- GPU from here on
    import torch
    import sparse_graph_attention_02_amd as ga
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    plan = ga.Plan(ip, ix, light_max_deg=args.light, hub_min_deg_exclusive=args.hub,
                   hub_chunk=args.chunk, build_csc=w.backward, feature_slices=args.slices,
                   col_hub_min_deg_exclusive=args.col_hub, col_hub_chunk=args.col_chunk,
                   xcd_split_min_deg_exclusive=args.xcd_split,
                   col_xcd_split_min_deg_exclusive=args.col_xcd_split)
    plan_host_s = time.perf_counter() - t0
    plan.upload("cuda")
    torch.cuda.synchronize()
    plan_s = time.perf_counter() - t0
    info = plan.info()
    tens = [to_dev(x) for x in feats]
    tdo = to_dev(dout) if dout is not None else None
    stream = torch.cuda.current_stream()

    # copy-kernel bandwidth on this device (the measured ceiling next to the 8 TB/s spec;
    # also the calibration kernel of the traffic counters)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        ga.copy_probe(dst, src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        ga.copy_probe(dst, src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    red = w.score in REDUCTIONS
    vt = tens[1] if w.score == "gatv2" else tens[0] if red else tens[2]
    out = torch.empty_like(vt)
    lse = torch.empty((N, H), dtype=torch.float32, device="cuda")
    fws = torch.empty(max(plan.fwd_workspace_bytes(H, d), 1), dtype=torch.uint8, device="cuda")
    if red:
        arg = torch.empty(vt.shape, dtype=torch.int32, device="cuda")
        slot = torch.empty(vt.shape, dtype=ga.reduce_slot_dtype(plan), device="cuda")
        fws = torch.empty(max(int(capi_ws("graph_attn_reduce_fwd_workspace_bytes", plan,
                                          H * d)), 1), dtype=torch.uint8, device="cuda")
        if w.backward:
            dq = torch.empty_like(vt)
            bws = torch.empty(max(int(capi_ws("graph_attn_reduce_bwd_workspace_bytes", plan,
                                              H * d)), 1), dtype=torch.uint8, device="cuda")
    elif w.backward and w.score == "gatv2":
        dq, dk = torch.empty_like(vt), torch.empty_like(vt)
        dv = torch.empty((H, d), dtype=torch.float32, device="cuda")
        bws = torch.empty(ga.bwd_gatv2_workspace_bytes(plan, vt.dtype, H, d), dtype=torch.uint8,
                          device="cuda")
    elif w.backward:
        # dot: dq, dk, dv like q, k, v; GAT-style: ds, dt like s, t and dv like v
        dq, dk, dv = (torch.empty_like(x) for x in tens)
        bws = torch.empty(plan.bwd_workspace_bytes(H, d), dtype=torch.uint8, device="cuda")

    def forward():
        if red:
            ga.reduce_fwd(plan, tens[0], op=w.score, out=out, arg=arg, slot=slot, workspace=fws)
        elif w.score == "gatv2":
            ga.fwd_gatv2(plan, *tens, scale=scale, out=out, lse=lse, workspace=fws)
        else:
            ga.fwd(plan, *tens, score=w.score, scale=scale, out=out, lse=lse, workspace=fws)

    def backward():
        """The backward alone, from what the last forward saved (lse, or the slots)."""
        if red:
            ga.reduce_bwd(plan, None, tdo, slot=slot, dx=dq, workspace=bws)
        elif w.score == "gatv2":
            ga.bwd_gatv2(plan, *tens, tdo, lse, scale=scale, dxd=dq, dxs=dk, dattn=dv,
                         workspace=bws)
        else:
            ga.bwd(plan, *tens, tdo, lse, score=w.score, scale=scale, dq=dq, dk=dk, dv=dv,
                   workspace=bws)

    def step(with_backward=w.backward):
        forward()
        if with_backward:
            backward()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(fn, k):
        ga.timers(enable=True, reset=True)
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(k):
            fn()
        z.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(z) / k
        kt = ga.timers(enable=False, reset=True)
        return ms, kt

    # the library's kernel timers take their hipEvents from a pool that grows on first use;
    # one untimed pass with the timers on fills it, so that no timed region pays for event
    # creation (which short kernels cannot hide)
    timed(step, args.steps)
    ms_step, kt = timed(step, args.steps)
    ms_fwd, kt_fwd = timed(lambda: step(False), args.steps)

    def per_step(fn, k):
        """Each of k launches bracketed by its own pair of events on the launch stream:
        median, p10 and p90 in ms."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(k)]
        torch.cuda.synchronize()
        for a, z in ev:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(z) for a, z in ev])
        return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
                "p90": float(np.percentile(t, 90))}

    dist_step = per_step(step, args.steps)
    dist_fwd = per_step(lambda: step(False), args.steps)
    if w.backward:           # the last forward's lse / slots are in place
        ms_bwd, _ = timed(backward, args.steps)
        dist_bwd = per_step(backward, args.steps)
    # peak memory of one step above what is already allocated (inputs, outputs, plan and
    # workspaces are allocated before the timed region; a step allocates nothing)
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    step_peak_extra = torch.cuda.max_memory_allocated() - base_alloc

    # floors: the passes' loads alone, over the same plan's work lists (gather-only probes)
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    probes = {}
    if red:
        probes["reduce_fwd_main"] = ("rows", lambda: ga.gather_probe(plan, tens[0], sink=sink))
    elif w.score == "gatv2":
        probes["fwd_main"] = ("rows", lambda: ga.gather_probe(plan, tens[1], row_a=tens[0],
                                                              sink=sink))
    elif w.score == "gat":
        probes["fwd_main"] = ("rows", lambda: ga.gather_probe(plan, tens[2], sink=sink))
    else:
        probes["fwd_main"] = ("rows", lambda: ga.gather_probe(plan, tens[1], tens[2],
                                                              row_a=tens[0], sink=sink))
    if w.backward and not red:
        rec = torch.zeros((N, H, 2), dtype=torch.float32, device="cuda")
        if w.score == "dot":
            probes["bwd_dq_main"] = ("rows", lambda: ga.gather_probe(
                plan, tens[1], tens[2], row_a=tens[0], row_b=tdo, sink=sink))
            probes["bwd_dkdv_main"] = ("cols", lambda: ga.gather_probe_cols(
                plan, tdo, q=tens[0], record=rec, k=tens[1], v=tens[2], sink=sink))
        elif w.score == "gatv2":
            probes["bwd_gatv2_cols_main"] = ("cols", lambda: ga.gather_probe_cols(
                plan, tdo, q=tens[0], record=rec, k=tens[1], sink=sink))
    floor_ms = {}
    for name, (kind, fn) in probes.items():
        fn()
        pm, pk = timed(fn, args.steps)
        floor_ms[name] = next(t / n for n, t in pk.values())

    # gather ceiling: uniformly random rows of the workload's row width from tables of
    # growing size (L2-, MALL- and HBM-resident), the memory hierarchy's gather rate
    ceiling = None
    row_bytes = H * d * b
    if args.ceiling_gathers > 0 and row_bytes in (64, 128, 256, 512, 1024):
        sizes = [2 << 20, 64 << 20, 512 << 20, 2 << 30, 8 << 30]
        table = torch.zeros(sizes[-1], dtype=torch.uint8, device="cuda")
        ceiling = {"row_bytes": row_bytes, "gathers": args.ceiling_gathers, "tables": []}
        for sz in sizes:
            fn = lambda: ga.gather_probe_random(table, row_bytes, args.ceiling_gathers,
                                                table_rows=sz // row_bytes, sink=sink)
            fn()
            pm, _ = timed(fn, 5)
            gbps = args.ceiling_gathers * row_bytes / (pm * 1e-3) / 1e9
            ceiling["tables"].append({"table_bytes": sz, "ms": pm, "GBps": gbps})
        del table
    torch.cuda.synchronize()
    if int(sink.sum()) != 0:
        raise RuntimeError("a probe wrote its sink")

    main_fwd = "reduce_fwd_main" if red else "fwd_main"
    node_order = args.order
    kernels = {}
    for name, (launches, tot) in kt.items():
        per = tot / launches
        kernels[name] = {"launches_per_step": launches / args.steps, "avg_ms": per,
                         "share": tot / (ms_step * args.steps)}
        lb = algorithmic_bytes(name, N, E, H, d, b, w.score)
        cb = compulsory_bytes(name, N, E, H, d, b, w.score)
        tb = measured_traffic(w.name, name, info, node_order)
        if lb is not None:
            kernels[name].update(logical_bytes=lb, logical_GBps=_rates(lb, per),
                                 compulsory_bytes=cb, compulsory_GBps=_rates(cb, per))
        if tb is not None:
            kernels[name].update(l2_miss_bytes=tb, l2_miss_GBps=_rates(tb, per))
        if name in floor_ms:
            kernels[name].update(floor_ms=floor_ms[name], over_floor=per / floor_ms[name])
    dom = max((k for k in kernels if "logical_bytes" in kernels[k]),
              key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches_per_step"])
    dk_ = kernels[dom]
    up = dk_.get("l2_miss_GBps")

    def bracket(names, ms):
        """Compulsory (lower) and L2-miss (upper) bounds of the HBM rate of the kernels
        `names` over `ms` per step, and their fractions of the peak (None when a kernel's
        counters are not on record)."""
        comp = sum(compulsory_bytes(k, N, E, H, d, b, w.score) or 0 for k in names
                   if k in kernels)
        miss = [kernels[k].get("l2_miss_bytes") for k in names if k in kernels]
        lo = _rates(comp, ms)
        hi = _rates(sum(miss), ms) if miss and None not in miss else None
        return {"hbm_GBps_lower": lo, "frac_lower": lo / HBM_PEAK_GBPS,
                "hbm_GBps_upper": hi, "frac_upper": None if hi is None else hi / HBM_PEAK_GBPS}

    fwd_names = [k for k in kt_fwd]
    tot_bytes = step_bytes(N, E, H, d, b, w.backward, w.score)
    fwd_bytes = step_bytes(N, E, H, d, b, False, w.score)
    fwd_main_ms = kt_fwd[main_fwd][1] / kt_fwd[main_fwd][0]
    rec = {
        "metric": "fused graph-attn fwd/bwd edges/sec + achieved HBM GB/s (% of MI355X peak)",
        "value": E / (ms_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_ms_distribution": dist_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "graph": w.graph, "nodes": N, "edges": E, "heads": H, "dim": d,
            "score": w.score, "step": "forward+backward" if w.backward else "forward",
            "node_order": node_order,
            "plan": {k: info[k] for k in PLAN_KEYS},
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "kernel": dom, "achieved": up, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": None if up is None else up / HBM_PEAK_GBPS,
            "traffic": dk_.get("l2_miss_bytes"),
            "basis": "achieved = the kernel's L2-miss bytes per launch (rocprofv3 FETCH_SIZE "
                     "and WRITE_SIZE, calibrated on the copy kernel; committed counter runs of "
                     "these kernel sources and this plan) / its average launch time here: an "
                     "upper bound on its HBM rate, as the MALL may serve misses",
            "compulsory_GBps": dk_["compulsory_GBps"],
            "frac_compulsory": dk_["compulsory_GBps"] / HBM_PEAK_GBPS,
            "compulsory_basis": "every operand and output row moved once: a lower bound on "
                                "its HBM rate",
            "logical_GBps": dk_["logical_GBps"],
            "logical_basis": "one read of every gathered row per edge (re-gathers served by "
                             "L2 and MALL included): a work rate, not a memory fraction",
            "floor_ms": dk_.get("floor_ms"), "over_floor": dk_.get("over_floor"),
        },
        "cpu_baseline": cpu,
        "step": dict(bracket(list(kt), ms_step),
                     logical_GBps=_rates(tot_bytes, ms_step),
                     frac_of_copy_probe_logical=_rates(tot_bytes, ms_step) / copy_gbps),
        "fwd": dict({"ms": ms_fwd, "ms_distribution": dist_fwd,
                     "edges_per_s": E / (ms_fwd * 1e-3), "main_ms": fwd_main_ms,
                     "logical_GBps": _rates(fwd_bytes, ms_fwd)},
                    **bracket(fwd_names, ms_fwd),
                    note="the forward alone; the bracket is its HBM rate between the "
                         "compulsory bytes and the L2-miss bytes of its kernels"),
        "bwd": (dict({"ms": ms_bwd, "ms_distribution": dist_bwd,
                      "edges_per_s": E / (ms_bwd * 1e-3),
                      "logical_GBps": _rates(tot_bytes - fwd_bytes, ms_bwd)},
                     **bracket([k for k in kt if k not in kt_fwd], ms_bwd),
                     note="the backward alone, timed after a forward")
                if w.backward else None),
        "floors": {k: {"probe_ms": floor_ms[k], "kernel_ms": kernels[k]["avg_ms"],
                       "kernel_over_floor": kernels[k]["avg_ms"] / floor_ms[k],
                       "probe": probes[k][0]}
                   for k in floor_ms if k in kernels},
        "gather_ceiling": ceiling,
        "kernels": kernels,
        "copy_probe_GBps": copy_gbps,
        "plan_build_s": plan_host_s, "plan_build_and_upload_s": plan_s,
        "workspace_bytes": {"fwd": fws.numel(),
                            "bwd": (bws.numel() if w.backward else 0),
                            "edge_score_tensor_would_be": E * H * 4},
        "memory_bytes": {"plan_device": plan.device_bytes(),
                         "allocated_before_step": base_alloc,
                         "extra_peak_during_step": step_peak_extra},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
