"""The full-size parity checker (tests/fullsize.py) on the host, at a small size: fed the
oracle's own results rounded to bf16 it passes every tensor; a planted error in one
element of dk, of out or of lse is found, at its index, and fails that tensor alone."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import graphgen as gg
from oracle import attention as A
from tests import fullsize

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_child(spec, tmp_path):
    path = tmp_path / "spec.json"
    path.write_text(json.dumps(spec))
    r = subprocess.run([sys.executable, "-m", "tests.fullsize", str(path)], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.stdout.strip(), r.stderr
    return r.returncode, json.loads(r.stdout.strip().splitlines()[-1])


@pytest.fixture(scope="module")
def small_step(tmp_path_factory):
    d = tmp_path_factory.mktemp("fullsize")
    os.environ["GRAPHGEN_CACHE"] = str(d / "cache")
    try:
        w = gg.WORKLOADS["chunglu1m_train_bf16"]
        n = 2500
        ip, ix = gg.make_graph(w, n)
        q, k, v = gg.make_features(w, n)
        dout = gg.make_dout(w, n)
    finally:
        del os.environ["GRAPHGEN_CACHE"]
    scale = float(np.float32(1 / np.sqrt(w.dim)))
    out, lse = A.forward(ip, ix, q, k, v, "dot", scale)
    dq, dk, dv = A.backward(ip, ix, q, k, v, dout, scale)
    bf = lambda x: gg.f32_to_bf16_bits(x.astype(np.float32))
    res = {"out": bf(out), "lse": lse.astype(np.float32), "dq": bf(dq), "dk": bf(dk),
           "dv": bf(dv)}
    return d, n, scale, res


def _spec(d, n, scale, res, tmp_path):
    files = {}
    for k, x in res.items():
        files[k] = str(tmp_path / f"{k}.npy")
        np.save(files[k], x, allow_pickle=False)
    return {"workload": "chunglu1m_train_bf16", "n": n, "graph_cache": str(d / "cache"),
            "scale": scale, "train": True, "gpu": files}


def test_checker_passes_the_rounded_oracle(small_step, tmp_path):
    d, n, scale, res = small_step
    rc, out = _run_child(_spec(d, n, scale, res, tmp_path), tmp_path)
    assert rc == 0 and out["ok"], out
    assert set(out["tensors"]) == {"out", "lse", "dq", "dk", "dv"}
    assert out["tensors"]["dk"]["elements"] == n * 8 * 32
    assert out["workers"] == fullsize.workers()


@pytest.mark.parametrize("name,flat", [("dk", 12345), ("out", 777), ("lse", 4321)])
def test_checker_finds_a_planted_error(small_step, tmp_path, name, flat):
    d, n, scale, res = small_step
    bad = {k: v.copy() for k, v in res.items()}
    x = bad[name].reshape(-1)
    if name == "lse":
        x[flat] = np.float32(x[flat] + 1e-3 * max(1.0, abs(float(x[flat]))))
    else:
        val = float(A.widen(x[flat:flat + 1])[0])
        x[flat] = gg.f32_to_bf16_bits(np.array([val + 0.5 + abs(val)], np.float32))[0]
    rc, out = _run_child(_spec(d, n, scale, bad, tmp_path), tmp_path)
    assert rc == 1 and not out["ok"]
    t = out["tensors"]
    assert not t[name]["ok"] and t[name]["worst"][0][0] == flat
    assert all(t[k]["ok"] for k in t if k != name)


def test_balanced_blocks_tile_the_range():
    ptr = np.r_[0, np.cumsum(np.random.default_rng(2).integers(0, 50, 1000))]
    for k in (1, 7, 64, 5000):
        b = fullsize.balanced_blocks(ptr, k)
        assert b[0][0] == 0 and b[-1][1] == 1000
        assert all(x[1] == y[0] for x, y in zip(b[:-1], b[1:]))
    assert fullsize.balanced_blocks(np.zeros(1, np.int64), 4) == []


def _cache_inputs(d, w, n):
    os.environ["GRAPHGEN_CACHE"] = str(d / "cache")
    try:
        ip, ix = gg.make_graph(w, n)
        feats = gg.make_features(w, n)
        dout = gg.make_dout(w, n)
    finally:
        del os.environ["GRAPHGEN_CACHE"]
    return ip, ix, feats, dout


def _save_all(tmp_path, res):
    files = {}
    for k, x in res.items():
        files[k] = str(tmp_path / f"{k}.npy")
        np.save(files[k], x, allow_pickle=False)
    return files


@pytest.mark.parametrize("plant", [None, "dt"])
def test_checker_gat_training_step(tmp_path, plant):
    """fp32 GAT-style training step: the rounded oracle passes at the fp32 criterion; an
    error of 1e-3 in one dt element fails dt alone."""
    w = gg.WORKLOADS["chunglu100k_gat_train_f32"]
    n = 2000
    ip, ix, (s, t, v), dout = _cache_inputs(tmp_path, w, n)
    out, lse = A.forward(ip, ix, s, t, v, "gat", 1.0, float(np.float32(0.2)))
    ds, dt, dv = A.backward_gat(ip, ix, s, t, v, dout, 1.0, float(np.float32(0.2)))
    res = {"out": out.astype(np.float32), "lse": lse.astype(np.float32),
           "ds": ds.astype(np.float32), "dt": dt.astype(np.float32), "dv": dv.astype(np.float32)}
    if plant:
        res[plant].reshape(-1)[321] += np.float32(1e-3)
    spec = {"workload": w.name, "n": n, "graph_cache": str(tmp_path / "cache"), "scale": 1.0,
            "slope": float(np.float32(0.2)), "train": True, "gpu": _save_all(tmp_path, res)}
    rc, got = _run_child(spec, tmp_path)
    assert set(got["tensors"]) == {"out", "lse", "ds", "dt", "dv"}
    if plant is None:
        assert rc == 0 and got["ok"], got
    else:
        assert rc == 1 and not got["tensors"][plant]["ok"]
        assert got["tensors"][plant]["worst"][0][0] == 321
        assert all(x["ok"] for k, x in got["tensors"].items() if k != plant)


@pytest.mark.parametrize("plant", [None, "dattn", "dxs"])
def test_checker_gatv2_training_step(tmp_path, plant):
    """bf16 GATv2 training step: the rounded oracle passes (dattn summed from the row
    blocks' shares); a planted error in one dattn or dxs element fails that tensor alone."""
    w = gg.WORKLOADS["chunglu1m_gatv2_train_bf16"]
    n = 1500
    ip, ix, (xd, xs, a), dout = _cache_inputs(tmp_path, w, n)
    sl = float(np.float32(0.2))
    out, lse = A.forward_gatv2(ip, ix, xd, xs, a, 1.0, sl)
    dxd, dxs, da = A.backward_gatv2(ip, ix, xd, xs, a, dout, 1.0, sl)
    bf = lambda x: gg.f32_to_bf16_bits(x.astype(np.float32))
    res = {"out": bf(out), "lse": lse.astype(np.float32), "dxd": bf(dxd), "dxs": bf(dxs),
           "dattn": da.astype(np.float32)}
    if plant == "dattn":
        res["dattn"].reshape(-1)[5] += np.float32(0.5 + abs(res["dattn"].reshape(-1)[5]))
    elif plant == "dxs":
        x = res["dxs"].reshape(-1)
        x[999] = gg.f32_to_bf16_bits(np.array([float(A.widen(x[999:1000])[0]) + 1.0],
                                              np.float32))[0]
    spec = {"workload": w.name, "n": n, "graph_cache": str(tmp_path / "cache"), "scale": 1.0,
            "slope": sl, "train": True, "gpu": _save_all(tmp_path, res)}
    rc, got = _run_child(spec, tmp_path)
    assert set(got["tensors"]) == {"out", "lse", "dxd", "dxs", "dattn"}
    if plant is None:
        assert rc == 0 and got["ok"], got
    else:
        assert rc == 1 and not got["tensors"][plant]["ok"]
        assert all(x["ok"] for k, x in got["tensors"].items() if k != plant)


@pytest.mark.parametrize("plant", [None, "arg", "slot", "dx"])
def test_checker_max_pooling_training_step(tmp_path, plant):
    """Max pooling on an XCD-split plan: out, arg and slot compared exactly (slots as
    positions in the plan's regrouped rows), dx at the bf16 criterion by feature columns;
    a planted error in one element fails that tensor alone, at its index."""
    from oracle import reduction as R
    from sparse_graph_attention_02_amd import Plan
    w = gg.WORKLOADS["chunglu1m_max_train_bf16"]
    n = 1500
    ip, ix, (x,), dout = _cache_inputs(tmp_path, w, n)
    plan = Plan(ip, ix, light_max_deg=4, xcd_split_min_deg_exclusive=8,
                col_xcd_split_min_deg_exclusive=8)
    pix = plan.array("indices")
    assert not np.array_equal(pix, ix)            # rows were regrouped
    F = w.heads * w.dim
    out, arg = R.reduce_rows(ip, ix, x, np.arange(n), "max")
    slot = R.slots_of(ip, pix, np.arange(n), arg)
    dx = R.reduce_backward(arg, dout.reshape(n, F), n)
    res = {"out": gg.f32_to_bf16_bits(out.astype(np.float32)), "arg": arg.astype(np.int32),
           "slot": np.where(slot < 0, 0xFFFF, slot).astype(np.uint16),
           "dx": gg.f32_to_bf16_bits(dx.astype(np.float32))}
    if plant == "arg":
        res["arg"].reshape(-1)[4242] += 1
    elif plant == "slot":
        res["slot"].reshape(-1)[777] ^= 1
    elif plant == "dx":
        y = res["dx"].reshape(-1)
        y[1234] = gg.f32_to_bf16_bits(np.array([float(A.widen(y[1234:1235])[0]) + 1.0],
                                               np.float32))[0]
    files = _save_all(tmp_path, res)
    np.save(tmp_path / "plan_ix.npy", pix, allow_pickle=False)
    spec = {"workload": w.name, "n": n, "graph_cache": str(tmp_path / "cache"), "train": True,
            "gpu": files, "plan_indices": str(tmp_path / "plan_ix.npy")}
    rc, got = _run_child(spec, tmp_path)
    assert set(got["tensors"]) == {"out", "arg", "slot", "dx"}
    if plant is None:
        assert rc == 0 and got["ok"], got
    else:
        assert rc == 1 and not got["tensors"][plant]["ok"]
        assert got["tensors"][plant]["worst"][0][0] == {"arg": 4242, "slot": 777,
                                                         "dx": 1234}[plant]
        assert all(x["ok"] for k, x in got["tensors"].items() if k != plant)
