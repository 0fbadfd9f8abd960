"""Node tables past 4 GiB: the gathered rows of 4.4M-node fp32 tensors with 1 KB rows sit
at byte offsets beyond the 32-bit range, which the structured-buffer gathers (forward,
GATv2 row pass, min/max forward) and the plain 64-bit gathers (dQ, dK/dV and column
passes) must both reach.

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

from oracle import attention as A
from oracle import reduction as R
from sparse_graph_attention_02_amd import (Plan, bwd, bwd_gatv2, fwd, fwd_gatv2, reduce_bwd,
                                           reduce_fwd)
from tests.gpu_util import check, check_lse, host64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N = 4_400_000          # x 1024-byte rows = 4.5e9 bytes per tensor
H, D = 4, 64           # fp32: 256 features, 1 KB per row
HIGH = 4_200_000       # ids from here on sit past 4 GiB


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def graph():
    """CSR over N nodes: 3000 destination rows (some above HIGH) of degree 1..40, 20 of
    degree 300..600 and one of 5000; neighbours 60% from [HIGH, N), 40% from [0, N).
    Returns the CSR, the touched nodes S (sorted) and the compact CSR over S."""
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
    say(f"N {N} E {E} touched {S.size} ids above 4 GiB: {(ix >= HIGH).sum()} edges")
    return ip.astype(np.int32), ix, S, ipc, ixc


def _rows(rng, n, shape):
    return rng.standard_normal((n,) + shape, dtype=np.float32)


def _scatter(S, rows):
    """Zero device tensor [N, ...] with the given rows at ids S."""
    t = torch.zeros((N,) + rows.shape[1:], dtype=torch.float32, device="cuda")
    t[torch.from_numpy(S).cuda()] = torch.from_numpy(rows).cuda()
    return t


def _others(S, k=4096):
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
    ip, ix, S, ipc, ixc = graph
    kw = dict(xcd_split_min_deg_exclusive=64, col_xcd_split_min_deg_exclusive=64) if split \
        else {}
    plan = Plan(ip, ix, **kw).upload()
    rng = np.random.default_rng(11)
    q, k, v, dout = (_rows(rng, S.size, (H, D)) for _ in range(4))
    scale = float(np.float32(1 / math.sqrt(D)))
    tq, tk, tv, td = (_scatter(S, x) for x in (q, k, v, dout))
    out, lse = fwd(plan, tq, tk, tv, scale=scale)
    dq, dk, dv = bwd(plan, tq, tk, tv, td, lse, scale=scale)
    torch.cuda.synchronize()
    del tq, tk, tv, td
    ro, rl = A.forward(ipc, ixc, q, k, v, "dot", scale)
    rq, rk, rv = A.backward(ipc, ixc, q, k, v, dout, scale)
    St = torch.from_numpy(S).cuda()
    for name, g, r in (("out", out, ro), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        say(name, check(name, host64(g[St]), r, "f32"))
    check_lse("lse", host64(lse[St]), rl)
    o = _others(S)
    for name, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        _empty_rows(name, t, o)
    _empty_rows("lse", lse, o, -np.inf)
    del out, lse, dq, dk, dv, plan
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_gatv2_training_step_past_4gib(graph):
    ip, ix, S, ipc, ixc = graph
    plan = Plan(ip, ix).upload()
    rng = np.random.default_rng(12)
    xd, xs, dout = (_rows(rng, S.size, (H, D)) for _ in range(3))
    attn = (rng.standard_normal((H, D), dtype=np.float32) / np.float32(8.0))
    slope = float(np.float32(0.2))
    txd, txs, td = (_scatter(S, x) for x in (xd, xs, dout))
    ta = torch.from_numpy(attn).cuda()
    out, lse = fwd_gatv2(plan, txd, txs, ta, scale=1.0, neg_slope=slope)
    dxd, dxs, dattn = bwd_gatv2(plan, txd, txs, ta, td, lse, scale=1.0, neg_slope=slope)
    torch.cuda.synchronize()
    del txd, txs, td
    ro, rl = A.forward_gatv2(ipc, ixc, xd, xs, attn, 1.0, slope)
    rd, rs, ra = A.backward_gatv2(ipc, ixc, xd, xs, attn, dout, 1.0, slope)
    St = torch.from_numpy(S).cuda()
    for name, g, r in (("out", out, ro), ("dxd", dxd, rd), ("dxs", dxs, rs)):
        say(name, check(name, host64(g[St]), r, "f32"))
    check_lse("lse", host64(lse[St]), rl)
    say("dattn", check("dattn", host64(dattn), ra, "f32"))
    o = _others(S)
    for name, t in (("out", out), ("dxd", dxd), ("dxs", dxs)):
        _empty_rows(name, t, o)
    del out, lse, dxd, dxs, plan
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_max_pooling_step_past_4gib(graph):
    ip, ix, S, ipc, ixc = graph
    plan = Plan(ip, ix).upload()
    rng = np.random.default_rng(13)
    F = H * D
    x, dout = _rows(rng, S.size, (F,)), _rows(rng, S.size, (F,))
    tx, td = _scatter(S, x), _scatter(S, dout)
    out, arg, slot = reduce_fwd(plan, tx, op="max")
    dx = reduce_bwd(plan, None, td, slot=slot)
    torch.cuda.synchronize()
    del tx, td
    rows = np.arange(S.size)
    ro, ra = R.reduce_rows(ipc, ixc, x, rows, "max")
    rs = R.slots_of(ipc, ixc, rows, ra)
    rdx = R.reduce_backward(ra, dout.reshape(S.size, F), S.size)
    St = torch.from_numpy(S).cuda()
    go = out[St].cpu().numpy()
    assert np.array_equal(go.view(np.uint32), ro.astype(np.float32).view(np.uint32)), "out"
    ga = arg[St].cpu().numpy().astype(np.int64)
    assert np.array_equal(ga, np.where(ra < 0, -1, S[np.maximum(ra, 0)])), "arg"
    gs = slot[St].cpu().numpy()
    gs = (gs.view(np.uint16).astype(np.int64) if gs.dtype == np.int16
          else gs.astype(np.int64))
    gs[gs == (0xFFFF if slot.dtype == torch.int16 else -1)] = -1
    assert np.array_equal(gs, rs), "slot"
    say("dx", check("dx", host64(dx[St]), rdx, "f32"))
    o = _others(S)
    _empty_rows("out", out, o)
    _empty_rows("dx", dx, o)
    _empty_rows("arg", arg.float(), o, -1.0)
    del out, arg, slot, dx, plan
    torch.cuda.empty_cache()
