"""Benchmark of the fused CSR graph-attention layer on one MI355X.

A step is one training step of the layer on the 1M-node Chung-Lu workload (gamma 2.1,
average in-degree 50 plus self-loops, H = 8, d = 32, bf16 with fp32 accumulation): the
forward (scores -> online softmax -> weighted V, saving the per-row log-sum-exp), then
the backward (dQ over CSR, dK/dV over the cached transpose).  The graph plan is built
once per graph, before the timed region, as the method caches graph metadata.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]

Prints one JSON line.  ``value`` is edges/s of the whole step (E / step time) with
inputs resident in HBM; ``roofline`` is the dominant kernel's algorithmic bytes per
launch over its measured average duration (HIP events recorded by the library on the
launch stream); ``cpu_baseline`` is the fp64 oracle timed on this host on a time-boxed
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# XCD split thresholds of the attention workloads' plans (rows, transpose columns): a sweep
# on the 1M-node training step gave 19.19 ms unsplit, 17.54 ms at 256 / 1024, 17.71 ms at
# 512 / 512 and 18.31 ms at 128 / 128 (chunk partials outgrow the L2 gain below ~256)
XCD_SPLIT_ROWS, XCD_SPLIT_COLS = 256, 1024
# the min / max reduction's chunk partials (value, id, edge) are larger, so its merge is
# dearer: 7.85 ms unsplit, 7.56 ms at 256 / 1024, 7.40 ms at 512 / 512 on the 1M max step
XCD_SPLIT_REDUCE = 512


# ---------------------------------------------------------------- algorithmic bytes

def algorithmic_bytes(kernel, N, E, H, d, b, score="dot"):
    """Bytes a launch must move at minimum: the CSR (or transpose) once, one read of each
    gathered row per edge, each per-node operand once and each output once."""
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
    cores = min(16, len(os.sched_getaffinity(0)))
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
        "value": e / longest, "unit": "edges/s", "cores": cores, "kind": "oracle",
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


def source_digest():
    """Digest of the device sources (kernels and the headers they include); host-only
    files (the planner, the C-ABI layer) do not change what the counters measured."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_graph_attention_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel sources (else None)."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = t.get(workload, {}).get(kernel)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the fused layer is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    w = gg.WORKLOADS[args.workload]
    args.xcd_split, args.col_xcd_split = xcd_split_of(w, args.xcd_split, args.col_xcd_split)
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
        print(f"[bench] cpu oracle: {cpu['value']:.3g} edges/s on {cpu['cores']} cores",
              file=sys.stderr, flush=True)

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

    # copy-kernel bandwidth on this device (the measured ceiling next to the 8 TB/s spec)
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
    # gather floor: the forward's neighbour gathers alone (same graph, same lane pattern)
    sink = torch.empty(1024, dtype=torch.uint8, device="cuda")
    # dot gathers two rows per edge (K_j, V_j); the other forms one (the probe then loads
    # the same row twice and the second load hits in cache)
    kv = (tens[1], tens[2]) if w.score == "dot" else (vt, vt)
    ga.gather_probe(plan, *kv, sink=sink)
    ms_gather, _ = timed(lambda: ga.gather_probe(plan, *kv, sink=sink), args.steps)
    rows_per_edge = 2 if w.score == "dot" else 1
    gather_bytes = rows_per_edge * E * H * d * b + 4 * E
    main_fwd = "reduce_fwd_main" if red else "fwd_main"

    kernels = {}
    for name, (launches, tot) in kt.items():
        per = tot / launches
        ab = algorithmic_bytes(name, N, E, H, d, b, w.score)
        kernels[name] = {"launches_per_step": launches / args.steps, "avg_ms": per,
                         "share": tot / (ms_step * args.steps)}
        if ab is not None:
            kernels[name].update(algorithmic_bytes=ab, GBps=ab / (per * 1e-3) / 1e9)
    dom = max((k for k in kernels if "algorithmic_bytes" in kernels[k]),
              key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches_per_step"])
    dk_ = kernels[dom]
    ach = dk_["GBps"]
    traffic = measured_traffic(w.name, dom)
    fwd_bytes = step_bytes(N, E, H, d, b, False, w.score)
    tot_bytes = step_bytes(N, E, H, d, b, w.backward, w.score)
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
            "node_order": args.order,
            "plan": {k: info[k] for k in ("light_max_deg", "hub_min_deg_exclusive", "hub_chunk",
                                          "n_row_light", "n_row_medium", "n_row_hub",
                                          "n_row_chunks", "n_col_hub", "n_col_chunks",
                                          "max_in_degree", "max_out_degree", "rows_sorted",
                                          "feature_slices", "col_hub_min_deg_exclusive",
                                          "col_hub_chunk", "xcd_split_min_deg_exclusive",
                                          "col_xcd_split_min_deg_exclusive", "n_row_sched",
                                          "n_col_sched")},
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS, "traffic": traffic},
        "cpu_baseline": cpu,
        "step_GBps_algorithmic": tot_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": tot_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "step_frac_of_copy_probe": tot_bytes / (ms_step * 1e-3) / 1e9 / copy_gbps,
        "fwd": {"ms": ms_fwd, "ms_distribution": dist_fwd, "edges_per_s": E / (ms_fwd * 1e-3),
                "GBps_algorithmic": fwd_bytes / (ms_fwd * 1e-3) / 1e9,
                "frac_of_peak": fwd_bytes / (ms_fwd * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "frac_of_copy_probe": fwd_bytes / (ms_fwd * 1e-3) / 1e9 / copy_gbps,
                "fwd_main_ms": fwd_main_ms},
        "bwd": ({"ms": ms_bwd, "ms_distribution": dist_bwd, "edges_per_s": E / (ms_bwd * 1e-3),
                 "GBps_algorithmic": (tot_bytes - fwd_bytes) / (ms_bwd * 1e-3) / 1e9,
                 "frac_of_peak": (tot_bytes - fwd_bytes) / (ms_bwd * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "frac_of_copy_probe": (tot_bytes - fwd_bytes) / (ms_bwd * 1e-3) / 1e9 / copy_gbps,
                 "note": "the backward alone, timed after a forward"}
                if w.backward else None),
        "gather_floor": {
            "ms": ms_gather, "GBps_algorithmic": gather_bytes / (ms_gather * 1e-3) / 1e9,
            "fwd_main_frac_of_floor": ms_gather / fwd_main_ms,
            "rows_per_edge": rows_per_edge,
            "note": "the source rows of every edge gathered with the forward's lane pattern "
                    "and no arithmetic (graph_attn_gather_probe); the memory system's floor "
                    "for the forward's gathers on this graph"},
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
