"""GPU parity on plans that regroup long rows / columns by neighbour id mod 8 and schedule
their chunks to the matching XCD (xcd_split_min_deg_exclusive): the dot forward and
backward, the GAT-style and GATv2 layers, against the fp64 oracle on the caller's CSR
(the regrouping must not change results beyond rounding). The full-size cases in the
bench's split configuration are in test_gpu_parity.py (FULL_PLANS).
"""
import math

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A
from sparse_graph_attention_02_amd import Plan, bwd, fwd
from tests.gpu_util import check, check_lse, dev, host64
from tests.test_gpu_parity import (GEOMS, bwd_case, f32, fwd_parity,
                                   gat_bwd_case, gatv2_bwd_case, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _fwd_ok(tag, ip, ix, q, k, v, out, lse, dtype, rows=None):
    scale = f32(1 / math.sqrt(q.shape[2]))
    rows = np.arange(ip.size - 1) if rows is None else np.asarray(rows)
    ro, rl = A.forward_rows(ip, ix, q, k, v, rows, "dot", scale, f32(0.2))
    rt = torch.from_numpy(rows).cuda()
    check(f"{tag} out", host64(out[rt]), ro, dtype)
    check_lse(f"{tag} lse", host64(lse[rt]), rl)


def _scheduled(plan):
    info = plan.info()
    assert info["n_row_sched"] > 0 and info["n_row_sched"] % 32 == 0
    assert info["n_col_sched"] > 0 and info["n_col_sched"] % 32 == 0
    return info


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [8, 1000])
def test_split_dot_forward_backward_every_element(dtype, chunk):
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 5000
    ip, ix = gg.make_graph(w, n=n)
    rng = np.random.default_rng(71)
    feats = [rng.standard_normal((n, 8, 32)).astype(np.float32) for _ in range(4)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    plan, r = bwd_case(f"split bwd chunglu5k {dtype} chunk {chunk}", ip, ix, *feats, dtype,
                       light_max_deg=8, hub_min_deg_exclusive=256, hub_chunk=chunk,
                       xcd_split_min_deg_exclusive=16)
    _fwd_ok("split fwd chunglu5k", ip, ix, *feats[:3], r[0], r[1], dtype)
    info = _scheduled(plan)
    assert info["n_row_chunks"] > 8 * info["n_row_hub"] // 2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_split_backward_geometries(G, LH, dtype):
    """Dot forward and backward on every element for every compiled geometry, with every
    row and column above 12 edges split (and a row hub and a column hub in many chunks)."""
    eb = 4 if dtype == "f32" else 2
    H, d = G // LH, LH * 16 // eb
    rng = np.random.default_rng(G * 7 + LH)
    n = 300
    src = np.r_[rng.integers(0, n, 2500), np.full(600, 5)]
    dst = np.r_[rng.integers(0, n, 2500), rng.integers(0, n, 600)]
    dst[:500] = 9
    ip, ix = gg.csr_from_edges(n, src, dst)
    feats = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(4)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    plan, r = bwd_case(f"split bwd G{G} LH{LH} {dtype}", ip, ix, *feats, dtype, light_max_deg=4,
                       hub_min_deg_exclusive=40, hub_chunk=16, xcd_split_min_deg_exclusive=12)
    _fwd_ok(f"split fwd G{G} LH{LH}", ip, ix, *feats[:3], r[0], r[1], dtype)
    _scheduled(plan)


def test_split_one_edge_chunks_and_empty_rows():
    """Every row / column of more than one edge split, chunks of one edge; empty rows."""
    rng = np.random.default_rng(72)
    n, H, d = 400, 2, 32
    ip, ix = gg.csr_from_edges(n, rng.integers(0, n, 3000), rng.integers(0, 300, 3000))
    feats = [gg.f32_to_bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
             for _ in range(4)]
    plan, (out, lse, dq, dk, dv) = bwd_case("split one-edge chunks", ip, ix, *feats, "bf16",
                                            light_max_deg=1, hub_min_deg_exclusive=1,
                                            hub_chunk=1, xcd_split_min_deg_exclusive=1)
    _fwd_ok("split fwd one-edge chunks", ip, ix, *feats[:3], out, lse, "bf16")
    _scheduled(plan)
    empty = torch.from_numpy(np.flatnonzero(np.diff(ip) == 0)).cuda()
    assert empty.numel() > 0 and torch.all(dq[empty] == 0) and torch.all(out[empty] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_gat_and_gatv2_every_element(dtype):
    """GAT-style and GATv2 forward and backward on a split plan: the forwards run the XCD
    schedule, the backward passes the chunks in order; all against the oracle."""
    rng = np.random.default_rng(73)
    n, H, d = 2000, 4, 32
    src = np.r_[rng.integers(0, n, 24_000), np.full(2000, 11)]
    dst = np.r_[rng.integers(0, n, 24_000), rng.integers(0, n, 2000)]
    dst[:3000] = 7
    ip, ix = gg.csr_from_edges(n, src, dst)
    s = rng.standard_normal((n, H)).astype(np.float32)
    t = rng.standard_normal((n, H)).astype(np.float32)
    v, do, xd, xs = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(4))
    a = (rng.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        v, do, xd, xs = (gg.f32_to_bf16_bits(x) for x in (v, do, xd, xs))
    kw = dict(light_max_deg=4, hub_min_deg_exclusive=512, hub_chunk=64,
              xcd_split_min_deg_exclusive=10)
    plan, _ = gat_bwd_case(f"split gat bwd {dtype}", ip, ix, s, t, v, do, dtype, scale=1.3,
                           slope=0.1, **kw)
    _scheduled(plan)
    fwd_parity(f"split gat fwd {dtype}", ip, ix, s, t, v, dtype, score="gat", scale=1.3,
               neg_slope=0.1, **kw)
    plan, _ = gatv2_bwd_case(f"split gatv2 bwd {dtype}", ip, ix, xd, xs, a, do, dtype,
                             scale=1.1, slope=0.2, **kw)
    _scheduled(plan)


def test_split_agrees_with_unsplit_and_is_deterministic():
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 20_000
    ip, ix = gg.make_graph(w, n=n)
    q, k, v = gg.make_features(w, n=n)
    do = gg.make_dout(w, n=n)
    tq, tk, tv, td = dev(q), dev(k), dev(v), dev(do)
    say("split vs unsplit plan, chunglu20k bf16")
    res = []
    for xs in (0, 32, 32):
        plan = Plan(ip, ix, xcd_split_min_deg_exclusive=xs).upload()
        out, lse = fwd(plan, tq, tk, tv)
        res.append((out, lse, *bwd(plan, tq, tk, tv, td, lse)))
    torch.cuda.synchronize()
    for a, b in zip(res[1], res[2]):
        assert torch.equal(a, b)                    # run to run, bit for bit
    for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), res[0], res[1]):
        x, r = a.float(), b.float()
        rms = r.pow(2).mean().sqrt()
        tol = 1e-5 + 1e-4 * r.abs() if name == "lse" else 2e-2 * torch.maximum(r.abs(), rms)
        assert torch.all((x - r).abs() <= tol), name


@pytest.mark.parametrize("S", [2, 8])
def test_split_plan_overrides_feature_slices(S):
    """On a split plan the forward and the dQ pass run unsliced whatever feature_slices
    asks for; every result still matches the oracle."""
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 4000
    ip, ix = gg.make_graph(w, n=n)
    rng = np.random.default_rng(78 + S)
    feats = [gg.f32_to_bf16_bits(rng.standard_normal((n, 8, 32)).astype(np.float32))
             for _ in range(4)]
    plan, r = bwd_case(f"split plan, feature_slices {S}", ip, ix, *feats, "bf16",
                       light_max_deg=8, hub_min_deg_exclusive=512, hub_chunk=64,
                       xcd_split_min_deg_exclusive=24, feature_slices=S)
    _fwd_ok(f"split plan, feature_slices {S}", ip, ix, *feats[:3], r[0], r[1], "bf16")
    _scheduled(plan)
