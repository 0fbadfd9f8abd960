"""Node tables past 4 GiB: the gathered rows of 4.4M-node fp32 tensors with 1 KB rows, and
of 8.6M-node bf16 tensors with 512-byte rows, sit at byte offsets beyond the 32-bit range,
which the structured-buffer gathers (forward, GATv2 row pass, min/max forward) and the
plain 64-bit gathers (dQ, dK/dV and column passes) must both reach.

Only a few thousand destination rows have edges; most of their neighbours have ids above
4.2M (offsets above 4.3e9 bytes). The feature rows those edges touch are seeded on the
host and scattered into zero device tensors; the oracle runs on the compact subgraph of
the touched nodes (same edge order), and every other row must come out empty: out 0,
lse -inf, zero gradients.
"""
import math

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A
from oracle import reduction as R
from sparse_graph_attention_02_amd import (Plan, bwd, bwd_gatv2, fwd, fwd_gatv2, reduce_bwd,
                                           reduce_fwd)
from tests.gpu_util import check, check_lse, host64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# (dtype, nodes, heads, head dim, first id past 4 GiB): fp32 1 KB rows, bf16 512-byte rows
CONFIGS = [("f32", 4_400_000, 4, 64, 4_194_304), ("bf16", 8_600_000, 8, 32, 8_388_608)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", params=CONFIGS, ids=[c[0] for c in CONFIGS])
def graph(request):
    """CSR over N nodes: 3000 destination rows (some past 4 GiB) of degree 1..40, 20 of
    degree 300..600 and one of 5000; neighbours 60% from the ids past 4 GiB, 40% from all.
    Returns the config, the CSR, the touched nodes S (sorted) and the compact CSR over S."""
    dt, N, H, D, first = request.param
    HIGH = first + 10_000
    rng = np.random.default_rng(20261203)
    dst = np.unique(np.concatenate([rng.choice(N, 2900, replace=False),
                                    rng.integers(HIGH, N, 100)]))
    deg = rng.integers(1, 41, dst.size)
    big = rng.choice(dst.size, 21, replace=False)
    deg[big[:20]] = rng.integers(300, 601, 20)
    deg[big[20]] = 5000
    counts = np.zeros(N, np.int64)
    counts[dst] = deg
    ip = np.zeros(N + 1, np.int64)
    np.cumsum(counts, out=ip[1:])
    E = int(ip[-1])
    hi = rng.random(E) < 0.6
    ix = np.where(hi, rng.integers(HIGH, N, E), rng.integers(0, N, E)).astype(np.int32)
    S = np.unique(np.concatenate([dst, ix]))
    # compact CSR over S, rows in S order, each row's edges in the original order
    pos = np.searchsorted(S, dst)
    cc = np.zeros(S.size, np.int64)
    cc[pos] = deg
    ipc = np.zeros(S.size + 1, np.int64)
    np.cumsum(cc, out=ipc[1:])
    ixc = np.searchsorted(S, ix).astype(np.int64)
    assert ipc[-1] == E and np.array_equal(S[ixc], ix)
    say(f"{dt} N {N} E {E} touched {S.size} neighbour rows past 4 GiB: {(ix >= first).sum()}")
    return (dt, N, H, D, HIGH), ip.astype(np.int32), ix, S, ipc, ixc


def _rows(rng, n, shape, dt):
    """Seeded rows: fp32, or bf16 bit patterns (uint16)."""
    x = rng.standard_normal((n,) + shape, dtype=np.float32)
    return x if dt == "f32" else gg.f32_to_bf16_bits(x)


def _scatter(N, S, rows):
    """Zero device tensor [N, ...] (fp32, or bf16 from uint16 bits) with the rows at ids S."""
    bf = rows.dtype == np.uint16
    t = torch.zeros((N,) + rows.shape[1:], dtype=torch.bfloat16 if bf else torch.float32,
                    device="cuda")
    src = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16) if bf \
        else torch.from_numpy(rows)
    t[torch.from_numpy(S).cuda()] = src.cuda()
    return t


def _others(N, HIGH, S, k=4096):
    """Sampled untouched ids, including the last node."""
    rng = np.random.default_rng(7)
    cand = np.concatenate([rng.integers(0, N, k), rng.integers(HIGH, N, k), [N - 1]])
    return np.setdiff1d(cand, S)


def _empty_rows(name, t, ids, value=0.0):
    x = host64(t[torch.from_numpy(ids).cuda()])
    assert np.all(x == value), f"{name}: untouched rows are not {value}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("split", [False, True], ids=["default-plan", "split-plan"])
def test_dot_training_step_past_4gib(graph, split):
    (dt, N, H, D, HIGH), ip, ix, S, ipc, ixc = graph
    kw = dict(xcd_split_min_deg_exclusive=64, col_xcd_split_min_deg_exclusive=64) if split \
        else {}
    plan = Plan(ip, ix, **kw).upload()
    rng = np.random.default_rng(11)
    q, k, v, dout = (_rows(rng, S.size, (H, D), dt) for _ in range(4))
    scale = float(np.float32(1 / math.sqrt(D)))
    tq, tk, tv, td = (_scatter(N, S, x) for x in (q, k, v, dout))
    out, lse = fwd(plan, tq, tk, tv, scale=scale)
    dq, dk, dv = bwd(plan, tq, tk, tv, td, lse, scale=scale)
    torch.cuda.synchronize()
    del tq, tk, tv, td
    ro, rl = A.forward(ipc, ixc, q, k, v, "dot", scale)
    rq, rk, rv = A.backward(ipc, ixc, q, k, v, dout, scale)
    St = torch.from_numpy(S).cuda()
    for name, g, r in (("out", out, ro), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        say(name, check(name, host64(g[St]), r, dt))
    check_lse("lse", host64(lse[St]), rl)
    o = _others(N, HIGH, S)
    for name, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        _empty_rows(name, t, o)
    _empty_rows("lse", lse, o, -np.inf)
    del out, lse, dq, dk, dv, plan
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_gat_training_step_past_4gib(graph):
    """GAT-style scores: s, t per node and head (fp32), V rows past 4 GiB."""
    (dt, N, H, D, HIGH), ip, ix, S, ipc, ixc = graph
    plan = Plan(ip, ix).upload()
    rng = np.random.default_rng(14)
    s_, t_ = (rng.standard_normal((S.size, H), dtype=np.float32) for _ in range(2))
    v, dout = (_rows(rng, S.size, (H, D), dt) for _ in range(2))
    slope = float(np.float32(0.2))
    ts, tt = _scatter(N, S, s_), _scatter(N, S, t_)
    tv, td = _scatter(N, S, v), _scatter(N, S, dout)
    out, lse = fwd(plan, ts, tt, tv, score="gat", scale=1.0, neg_slope=slope)
    ds, dtt, dv = bwd(plan, ts, tt, tv, td, lse, score="gat", scale=1.0, neg_slope=slope)
    torch.cuda.synchronize()
    del ts, tt, tv, td
    ro, rl = A.forward(ipc, ixc, s_, t_, v, "gat", 1.0, slope)
    rs, rt_, rv = A.backward_gat(ipc, ixc, s_, t_, v, dout, 1.0, slope)
    St = torch.from_numpy(S).cuda()
    for name, g, r, kind in (("out", out, ro, dt), ("ds", ds, rs, "f32"), ("dt", dtt, rt_, "f32"),
                             ("dv", dv, rv, dt)):
        say(name, check(name, host64(g[St]), r, kind))
    check_lse("lse", host64(lse[St]), rl)
    o = _others(N, HIGH, S)
    for name, t in (("out", out), ("ds", ds), ("dt", dtt), ("dv", dv)):
        _empty_rows(name, t, o)
    del out, lse, ds, dtt, dv, plan
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_gatv2_training_step_past_4gib(graph):
    (dt, N, H, D, HIGH), ip, ix, S, ipc, ixc = graph
    plan = Plan(ip, ix).upload()
    rng = np.random.default_rng(12)
    xd, xs, dout = (_rows(rng, S.size, (H, D), dt) for _ in range(3))
    attn = (rng.standard_normal((H, D), dtype=np.float32) / np.float32(8.0))
    slope = float(np.float32(0.2))
    txd, txs, td = (_scatter(N, S, x) for x in (xd, xs, dout))
    ta = torch.from_numpy(attn).cuda()
    out, lse = fwd_gatv2(plan, txd, txs, ta, scale=1.0, neg_slope=slope)
    dxd, dxs, dattn = bwd_gatv2(plan, txd, txs, ta, td, lse, scale=1.0, neg_slope=slope)
    torch.cuda.synchronize()
    del txd, txs, td
    ro, rl = A.forward_gatv2(ipc, ixc, xd, xs, attn, 1.0, slope)
    rd, rs, ra = A.backward_gatv2(ipc, ixc, xd, xs, attn, dout, 1.0, slope)
    St = torch.from_numpy(S).cuda()
    for name, g, r in (("out", out, ro), ("dxd", dxd, rd), ("dxs", dxs, rs)):
        say(name, check(name, host64(g[St]), r, dt))
    check_lse("lse", host64(lse[St]), rl)
    say("dattn", check("dattn", host64(dattn), ra, dt))
    o = _others(N, HIGH, S)
    for name, t in (("out", out), ("dxd", dxd), ("dxs", dxs)):
        _empty_rows(name, t, o)
    del out, lse, dxd, dxs, plan
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_max_pooling_step_past_4gib(graph):
    (dt, N, H, D, HIGH), ip, ix, S, ipc, ixc = graph
    plan = Plan(ip, ix).upload()
    rng = np.random.default_rng(13)
    F = H * D
    x, dout = _rows(rng, S.size, (F,), dt), _rows(rng, S.size, (F,), dt)
    tx, td = _scatter(N, S, x), _scatter(N, S, dout)
    out, arg, slot = reduce_fwd(plan, tx, op="max")
    dx = reduce_bwd(plan, None, td, slot=slot)
    torch.cuda.synchronize()
    del tx, td
    rows = np.arange(S.size)
    ro, ra = R.reduce_rows(ipc, ixc, x, rows, "max")
    rs = R.slots_of(ipc, ixc, rows, ra)
    rdx = R.reduce_backward(ra, dout.reshape(S.size, F), S.size)
    St = torch.from_numpy(S).cuda()
    go = out[St].cpu()
    if dt == "f32":
        assert np.array_equal(go.numpy().view(np.uint32),
                              ro.astype(np.float32).view(np.uint32)), "out"
    else:
        assert np.array_equal(go.view(torch.int16).numpy().view(np.uint16),
                              gg.f32_to_bf16_bits(ro.astype(np.float32))), "out"
    ga = arg[St].cpu().numpy().astype(np.int64)
    assert np.array_equal(ga, np.where(ra < 0, -1, S[np.maximum(ra, 0)])), "arg"
    gs = slot[St].cpu().numpy()
    gs = (gs.view(np.uint16).astype(np.int64) if gs.dtype == np.int16
          else gs.astype(np.int64))
    gs[gs == (0xFFFF if slot.dtype == torch.int16 else -1)] = -1
    assert np.array_equal(gs, rs), "slot"
    say("dx", check("dx", host64(dx[St]), rdx, dt))
    o = _others(N, HIGH, S)
    _empty_rows("out", out, o)
    _empty_rows("dx", dx, o)
    _empty_rows("arg", arg.float(), o, -1.0)
    del out, arg, slot, dx, plan
    torch.cuda.empty_cache()
