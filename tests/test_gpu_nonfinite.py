"""Non-finite features reach only what the plain definition lets them reach.

In the definition, a NaN or an infinity in node j's features enters only the rows whose
neighbour lists hold j (and, in the backward, what those rows feed). The kernels fold
several edges per step, and a step's spare slots still issue their loads with a zero
weight. These tests poison node 0 (NaN) and the last node (an infinite message) and require
every output the fp64 oracle computes as finite to match it within the usual criteria, on
the buffer-load path and on the 64-bit one (GRAPH_ATTN_WIDE_LOADS=1).

A second set puts each gathered table at the front of an allocation twice its size whose
second half is NaN. A read past a table's last row would find NaN there, so every output
must stay finite and match the oracle; the reads stay inside mapped memory either way.
"""
import math

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A
from sparse_graph_attention_02_amd import Plan, bwd, bwd_gatv2, fwd, fwd_gatv2
from tests.gpu_util import check, check_lse, dev, host64

pytestmark = pytest.mark.gpu

N, H, D = 2000, 2, 32
SLOPE = float(np.float32(0.2))
PLANS = {"default": {}, "small-bins": dict(light_max_deg=4, hub_min_deg_exclusive=9,
                                           hub_chunk=3)}
BF16_NAN, BF16_INF = np.uint16(0x7FC0), np.uint16(0x7F80)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


@pytest.fixture(params=["buffer", "wide"])
def path(request, monkeypatch):
    if request.param == "wide":
        monkeypatch.setenv("GRAPH_ATTN_WIDE_LOADS", "1")
    return request.param


def say(*a):
    print("[case]", *a, flush=True)


def graph():
    ip, ix = gg.make_graph(gg.WORKLOADS["er2k_dot_f32"])
    assert ip.size - 1 == N
    return ip, ix


def rows_of(dt, rng, shape):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dt == "f32" else gg.f32_to_bf16_bits(x)


def poison(x, node, kind):
    """Set node's row of a feature array (fp32, or bf16 bits) to NaN or +inf."""
    x = x.copy()
    if x.dtype == np.uint16:
        x[node] = BF16_NAN if kind == "nan" else BF16_INF
    else:
        x[node] = np.nan if kind == "nan" else np.inf
    return x


def inputs(score, dt, seed=3):
    """Seeded inputs with node 0 NaN in every gathered table and node N-1's message +inf."""
    rng = np.random.default_rng(seed)
    if score == "dot":
        a, b, v = (rows_of(dt, rng, (N, H, D)) for _ in range(3))
        return a, poison(b, 0, "nan"), poison(poison(v, 0, "nan"), N - 1, "inf")
    if score == "gat":
        s, t = (rng.standard_normal((N, H), dtype=np.float32) for _ in range(2))
        v = rows_of(dt, rng, (N, H, D))
        return s, poison(t, 0, "nan"), poison(poison(v, 0, "nan"), N - 1, "inf")
    xd, xs = (rows_of(dt, rng, (N, H, D)) for _ in range(2))
    attn = rng.standard_normal((H, D), dtype=np.float32) / np.float32(8)
    return xd, poison(poison(xs, 0, "nan"), N - 1, "inf"), attn


def finite_rows(*arrs):
    """Rows whose every element is finite in all the given [N, ...] arrays."""
    ok = np.ones(arrs[0].shape[0], bool)
    for x in arrs:
        ok &= np.isfinite(x.reshape(x.shape[0], -1)).all(axis=1)
    return ok


def compare(name, got, ref, dt, keep, min_keep=0.8):
    assert keep.mean() >= min_keep, f"{name}: only {keep.sum()} finite rows in the oracle"
    assert keep.sum() < keep.size, f"{name}: the poison reached no output"
    return check(name, host64(got)[keep], ref[keep], dt)


def forward_case(score, dt, a, b, v, plan_kw, tables=None):
    """GPU forward (tables: device tensors to use instead of uploading a, b, v) and oracle."""
    ip, ix = graph()
    plan = Plan(ip, ix, **plan_kw).upload()
    ta, tb, tv = tables or (dev(a), dev(b), dev(v))
    if score == "gatv2":
        out, lse = fwd_gatv2(plan, ta, tb, tv, scale=1.0, neg_slope=SLOPE)
        ro, rl = A.forward_gatv2(ip, ix, a, b, v, 1.0, SLOPE)
    else:
        scale = float(np.float32(1 / math.sqrt(D))) if score == "dot" else 1.0
        out, lse = fwd(plan, ta, tb, tv, score=score, scale=scale, neg_slope=SLOPE)
        ro, rl = A.forward(ip, ix, a, b, v, score, scale, SLOPE)
    torch.cuda.synchronize()
    return plan, out, lse, ro, rl


def nan_tailed(x):
    """Device tensor holding x in the first half of a NaN-filled allocation twice its size
    (a view of the first half is returned, with the allocation kept alive by it)."""
    t = dev(x)
    big = torch.full((2 * t.shape[0],) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype,
                     device=t.device)
    big[:t.shape[0]] = t
    return big[:t.shape[0]]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("score", ["dot", "gat", "gatv2"])
def test_reads_stay_inside_the_tables(score, dt, path):
    say("NaN past the tables", score, dt, path)
    ip, ix = graph()
    rng = np.random.default_rng(21)
    if score == "gatv2":
        a, b = rows_of(dt, rng, (N, H, D)), rows_of(dt, rng, (N, H, D))
        v = rng.standard_normal((H, D), dtype=np.float32) / np.float32(8)
        tables = (nan_tailed(a), nan_tailed(b), dev(v))
    else:
        if score == "dot":
            a, b = rows_of(dt, rng, (N, H, D)), rows_of(dt, rng, (N, H, D))
        else:
            a, b = (rng.standard_normal((N, H), dtype=np.float32) for _ in range(2))
        v = rows_of(dt, rng, (N, H, D))
        tables = (nan_tailed(a), nan_tailed(b), nan_tailed(v))
    dout = rows_of(dt, rng, (N, H, D))
    for plan_name, kw in PLANS.items():
        plan, out, lse, ro, rl = forward_case(score, dt, a, b, v, kw, tables)
        check(f"{plan_name} out", host64(out), ro, dt)
        check_lse(f"{plan_name} lse", host64(lse), rl)
        td = nan_tailed(dout)
        if score == "gatv2":
            g = bwd_gatv2(plan, *tables, td, lse, scale=1.0, neg_slope=SLOPE)
            r = A.backward_gatv2(ip, ix, a, b, v, dout, 1.0, SLOPE)
            names = ("dxd", "dxs", "dattn")
        elif score == "gat":
            g = bwd(plan, *tables, td, lse, score="gat", scale=1.0, neg_slope=SLOPE)
            r = A.backward_gat(ip, ix, a, b, v, dout, 1.0, SLOPE)
            names = ("ds", "dt", "dv")
        else:
            scale = float(np.float32(1 / math.sqrt(D)))
            g = bwd(plan, *tables, td, lse, scale=scale)
            r = A.backward(ip, ix, a, b, v, dout, scale)
            names = ("dq", "dk", "dv")
        torch.cuda.synchronize()
        for name, gt, rt in zip(names, g, r):
            kind = "f32" if name in ("ds", "dt") else dt
            check(f"{plan_name} {name}", host64(gt), rt, kind)


@pytest.mark.parametrize("plan_name", list(PLANS))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("score", ["dot", "gat", "gatv2"])
def test_forward_poison_stays_in_its_rows(score, dt, plan_name, path):
    say("forward", score, dt, plan_name, path)
    a, b, v = inputs(score, dt)
    with np.errstate(invalid="ignore", over="ignore"):
        _, out, lse, ro, rl = forward_case(score, dt, a, b, v, PLANS[plan_name])
    keep = finite_rows(ro, rl)
    say("finite rows", int(keep.sum()), "of", keep.size)
    compare("out", out, ro, dt, keep)
    check_lse("lse", host64(lse)[keep], rl[keep])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("score", ["dot", "gat", "gatv2"])
def test_backward_poison_stays_in_its_rows(score, dt, path):
    say("backward", score, dt, path)
    ip, ix = graph()
    a, b, v = inputs(score, dt)
    dout = rows_of(dt, np.random.default_rng(9), (N, H, D))
    plan = Plan(ip, ix, **PLANS["small-bins"]).upload()
    with np.errstate(invalid="ignore", over="ignore"):
        if score == "gatv2":
            out, lse = fwd_gatv2(plan, dev(a), dev(b), dev(v), scale=1.0, neg_slope=SLOPE)
            g = bwd_gatv2(plan, dev(a), dev(b), dev(v), dev(dout), lse, scale=1.0,
                          neg_slope=SLOPE)[:2]
            r = A.backward_gatv2(ip, ix, a, b, v, dout, 1.0, SLOPE)[:2]
            names = ("dxd", "dxs")
        elif score == "gat":
            out, lse = fwd(plan, dev(a), dev(b), dev(v), score="gat", scale=1.0,
                           neg_slope=SLOPE)
            g = bwd(plan, dev(a), dev(b), dev(v), dev(dout), lse, score="gat", scale=1.0,
                    neg_slope=SLOPE)
            r = A.backward_gat(ip, ix, a, b, v, dout, 1.0, SLOPE)
            names = ("ds", "dt", "dv")
        else:
            scale = float(np.float32(1 / math.sqrt(D)))
            out, lse = fwd(plan, dev(a), dev(b), dev(v), scale=scale)
            g = bwd(plan, dev(a), dev(b), dev(v), dev(dout), lse, scale=scale)
            r = A.backward(ip, ix, a, b, v, dout, scale)
            names = ("dq", "dk", "dv")
    torch.cuda.synchronize()
    for name, gt, rt in zip(names, g, r):
        kind = "f32" if name in ("ds", "dt") else dt
        keep = finite_rows(rt)
        say(name, "finite rows", int(keep.sum()), "of", keep.size)
        compare(name, gt, rt, kind, keep, min_keep=0.5)
