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
