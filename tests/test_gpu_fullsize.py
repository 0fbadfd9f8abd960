"""GPU parity on every element at full workload sizes, in the launch configuration bench.py
times (its XCD-split plans): the 1M-node Chung-Lu training step (out, lse, dq, dk, dv over
all 1M rows and columns; its forward is also the 1M forward workload's, checked bit for
bit on that workload's transpose-less plan), the R-MAT 2^21 forward (out, lse over all
2M rows), the 100k GAT-style fp32 training step (out, lse, ds, dt, dv), the 1M GATv2
training step (out, lse, dxd, dxs and the summed dattn) and the 1M max-pooling training
step (out, arg and slot exactly, dx).

The GPU results are saved to a directory and compared by a child process
(tests/fullsize.py) that runs the fp64 oracle over every row and column in forked worker
processes on the host, with the criteria of tests/gpu_util.py.
"""
import json
import math
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest
import torch

import bench
import graphgen as gg
from sparse_graph_attention_02_amd import (Plan, bwd, bwd_gatv2, fwd, fwd_gatv2, reduce_bwd,
                                           reduce_fwd)
from tests.gpu_util import dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


@pytest.fixture(scope="module")
def work_dir():
    """Generated inputs (GRAPHGEN_CACHE, shared with the checker) and saved GPU results, in
    shared memory when it has room."""
    base = "/dev/shm" if os.access("/dev/shm", os.W_OK) and \
        shutil.disk_usage("/dev/shm").free > (24 << 30) else None
    d = tempfile.mkdtemp(prefix="ga_fullsize_", dir=base)
    old = os.environ.get("GRAPHGEN_CACHE")
    os.environ["GRAPHGEN_CACHE"] = os.path.join(d, "cache")
    yield d
    if old is None:
        del os.environ["GRAPHGEN_CACHE"]
    else:
        os.environ["GRAPHGEN_CACHE"] = old
    shutil.rmtree(d, ignore_errors=True)


def say(*a):
    print("[case]", *a, flush=True)


def _save(d, name, t):
    x = t.detach().cpu()
    x = x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()
    path = os.path.join(d, f"gpu_{name}.npy")
    np.save(path, x, allow_pickle=False)
    return path


def _check_on_host(d, spec):
    path = os.path.join(d, "spec.json")
    with open(path, "w") as f:
        json.dump(spec, f)
    say("host oracle over every element:", spec["workload"])
    r = subprocess.run([sys.executable, "-m", "tests.fullsize", path], cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    lines = r.stdout.strip().splitlines()
    assert lines, f"checker printed nothing (rc {r.returncode}):\n{r.stderr[-3000:]}"
    res = json.loads(lines[-1])
    for name, t in res["tensors"].items():
        say(f"{name}: ok={t['ok']} elements={t['elements']} max_abs_err={t['max_abs_err']:.3g}"
            f" norm_rel_err={t['norm_rel_err']:.3g}"
            + (f" need_rms={t['need_rms']:.3g} rms={t['rms_ref']:.3g}" if "need_rms" in t
               else f" n_bad={t['n_bad']}"))
    say(f"workers {res['workers']}, oracle rows {res['rows_s']:.1f} s, total {res['total_s']:.1f} s")
    assert res["ok"], json.dumps(res["tensors"])
    return res


@pytest.mark.timeout(900)
def test_full_training_step_every_element_bench_plan(work_dir):
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    plan_kw = bench.bench_plan_kw(w)
    ip, ix = gg.make_graph(w)
    q, k, v = gg.make_features(w)
    dout = gg.make_dout(w)
    scale = float(np.float32(1 / math.sqrt(w.dim)))
    say("full chunglu1m training step, every element, plan", plan_kw, "E", ix.size)
    plan = Plan(ip, ix, **plan_kw).upload()
    assert plan.info()["n_row_sched"] > 0 and plan.info()["n_col_sched"] > 0
    tq, tk, tv, td = dev(q), dev(k), dev(v), dev(dout)
    out, lse = fwd(plan, tq, tk, tv, scale=scale)
    dq, dk, dv = bwd(plan, tq, tk, tv, td, lse, scale=scale)
    # the 1M forward workload runs on a plan of the same split without the transpose
    plan_fwd = Plan(ip, ix, build_csc=False,
                    **bench.bench_plan_kw(gg.WORKLOADS["chunglu1m_dot_bf16"])).upload()
    out2, lse2 = fwd(plan_fwd, tq, tk, tv, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    files = {n: _save(work_dir, n, t) for n, t in (("out", out), ("lse", lse), ("dq", dq),
                                                    ("dk", dk), ("dv", dv))}
    del tq, tk, tv, td, out, lse, dq, dk, dv, out2, lse2, plan, plan_fwd
    torch.cuda.empty_cache()
    _check_on_host(work_dir, {"workload": w.name, "graph_cache": os.environ["GRAPHGEN_CACHE"],
                              "scale": scale, "train": True, "gpu": files})


@pytest.mark.timeout(900)
def test_full_rmat21_forward_every_row_bench_plan(work_dir):
    w = gg.WORKLOADS["rmat21_dot_bf16"]
    plan_kw = bench.bench_plan_kw(w)
    ip, ix = gg.make_graph(w)
    q, k, v = gg.make_features(w)
    scale = float(np.float32(1 / math.sqrt(w.dim)))
    say("full rmat21 forward, every row, plan", plan_kw, "E", ix.size)
    plan = Plan(ip, ix, build_csc=False, **plan_kw).upload()
    assert plan.info()["max_in_degree"] > 100_000 and plan.info()["n_row_sched"] > 0
    out, lse = fwd(plan, dev(q), dev(k), dev(v), scale=scale)
    torch.cuda.synchronize()
    files = {"out": _save(work_dir, "out", out), "lse": _save(work_dir, "lse", lse)}
    del out, lse, plan
    torch.cuda.empty_cache()
    _check_on_host(work_dir, {"workload": w.name, "graph_cache": os.environ["GRAPHGEN_CACHE"],
                              "scale": scale, "train": False, "gpu": files})


@pytest.mark.timeout(900)
def test_full_gat_training_step_every_element_bench_plan(work_dir):
    w = gg.WORKLOADS["chunglu100k_gat_train_f32"]
    plan_kw = bench.bench_plan_kw(w)
    ip, ix = gg.make_graph(w)
    s, t, v = gg.make_features(w)
    dout = gg.make_dout(w)
    slope = float(np.float32(0.2))
    say("full chunglu100k GAT-style fp32 training step, every element, plan", plan_kw,
        "E", ix.size)
    plan = Plan(ip, ix, **plan_kw).upload()
    ts, tt, tv, td = dev(s), dev(t), dev(v), dev(dout)
    out, lse = fwd(plan, ts, tt, tv, score="gat", scale=1.0, neg_slope=slope)
    ds, dt, dv = bwd(plan, ts, tt, tv, td, lse, score="gat", scale=1.0, neg_slope=slope)
    torch.cuda.synchronize()
    files = {n: _save(work_dir, n, x) for n, x in (("out", out), ("lse", lse), ("ds", ds),
                                                    ("dt", dt), ("dv", dv))}
    del ts, tt, tv, td, out, lse, ds, dt, dv, plan
    torch.cuda.empty_cache()
    _check_on_host(work_dir, {"workload": w.name, "graph_cache": os.environ["GRAPHGEN_CACHE"],
                              "scale": 1.0, "slope": slope, "train": True, "gpu": files})


@pytest.mark.timeout(900)
def test_full_gatv2_training_step_every_element_bench_plan(work_dir):
    w = gg.WORKLOADS["chunglu1m_gatv2_train_bf16"]
    plan_kw = bench.bench_plan_kw(w)
    ip, ix = gg.make_graph(w)
    xd, xs, a = gg.make_features(w)
    dout = gg.make_dout(w)
    slope = float(np.float32(0.2))
    say("full chunglu1m GATv2 training step, every element, plan", plan_kw, "E", ix.size)
    plan = Plan(ip, ix, **plan_kw).upload()
    assert plan.info()["n_row_sched"] > 0 and plan.info()["n_col_sched"] > 0
    txd, txs, ta, td = dev(xd), dev(xs), dev(a), dev(dout)
    out, lse = fwd_gatv2(plan, txd, txs, ta, scale=1.0, neg_slope=slope)
    dxd, dxs, dattn = bwd_gatv2(plan, txd, txs, ta, td, lse, scale=1.0, neg_slope=slope)
    torch.cuda.synchronize()
    files = {n: _save(work_dir, n, x) for n, x in (("out", out), ("lse", lse), ("dxd", dxd),
                                                    ("dxs", dxs), ("dattn", dattn))}
    del txd, txs, ta, td, out, lse, dxd, dxs, dattn, plan
    torch.cuda.empty_cache()
    _check_on_host(work_dir, {"workload": w.name, "graph_cache": os.environ["GRAPHGEN_CACHE"],
                              "scale": 1.0, "slope": slope, "train": True, "gpu": files})


@pytest.mark.timeout(900)
def test_full_max_pooling_training_step_every_element_bench_plan(work_dir):
    w = gg.WORKLOADS["chunglu1m_max_train_bf16"]
    plan_kw = bench.bench_plan_kw(w)
    ip, ix = gg.make_graph(w)
    (x,) = gg.make_features(w)
    dout = gg.make_dout(w)
    say("full chunglu1m max-pooling training step, every element, plan", plan_kw,
        "E", ix.size)
    plan = Plan(ip, ix, **plan_kw).upload()
    assert plan.info()["n_row_sched"] > 0
    tx, td = dev(x), dev(dout)
    out, arg, slot = reduce_fwd(plan, tx, op="max")
    dx = reduce_bwd(plan, None, td, slot=slot)
    torch.cuda.synchronize()
    files = {n: _save(work_dir, n, t) for n, t in (("out", out), ("arg", arg), ("dx", dx))}
    # 16-bit slots are unsigned positions (all ones: the row is empty)
    sl = slot.cpu().numpy()
    files["slot"] = os.path.join(work_dir, "gpu_slot.npy")
    np.save(files["slot"], sl.view(np.uint16) if sl.dtype == np.int16 else sl,
            allow_pickle=False)
    pix = os.path.join(work_dir, "plan_indices.npy")
    np.save(pix, plan.array("indices"), allow_pickle=False)
    del tx, td, out, arg, slot, dx, plan
    torch.cuda.empty_cache()
    _check_on_host(work_dir, {"workload": w.name, "graph_cache": os.environ["GRAPHGEN_CACHE"],
                              "train": True, "gpu": files, "plan_indices": pix})
