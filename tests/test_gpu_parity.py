"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by
element on the same seeded inputs; at full workload sizes on sampled rows/columns.

Criteria are in tests/gpu_util.py. Each test prints the case it is about to run.
"""
import math

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A
from sparse_graph_attention_02_amd import Plan, bwd, fwd, graph_attention
from tests.gpu_util import check, check_lse, dev, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def say(*a):
    print("[case]", *a, flush=True)


def f32(x):
    return float(np.float32(x))


def run_fwd(ip, ix, a, b, v, score="dot", scale=None, neg_slope=0.2, **plan_kw):
    plan = Plan(ip, ix, **plan_kw).upload()
    out, lse = fwd(plan, dev(a), dev(b), dev(v), score=score, scale=scale, neg_slope=neg_slope)
    torch.cuda.synchronize()
    return plan, out, lse


def fwd_parity(tag, ip, ix, a, b, v, dtype, score="dot", scale=None, neg_slope=0.2, rows=None,
               **plan_kw):
    d = v.shape[2]
    if scale is None:
        scale = f32(1 / math.sqrt(d)) if score == "dot" else 1.0
    say(tag, "N", ip.size - 1, "E", ix.size, "H", v.shape[1], "d", d, dtype, score, plan_kw)
    plan, out, lse = run_fwd(ip, ix, a, b, v, score, scale, neg_slope, **plan_kw)
    rows = np.arange(ip.size - 1) if rows is None else np.asarray(rows)
    ro, rl = A.forward_rows(ip, ix, a, b, v, rows, score, scale, f32(neg_slope))
    rt = torch.from_numpy(rows).cuda()
    err = check(f"{tag} out", host64(out[rt]), ro, dtype)
    check_lse(f"{tag} lse", host64(lse[rt]), rl)
    return plan, out, lse, err


# ------------------------------------------------------------------ forward, small sizes

def test_er2k_f32_forward_every_row():
    w = gg.WORKLOADS["er2k_dot_f32"]
    ip, ix = gg.make_graph(w)
    q, k, v = gg.make_features(w)
    fwd_parity("er2k f32 dot", ip, ix, q, k, v, "f32")
    # same graph with every bin populated, including multi-chunk hubs
    fwd_parity("er2k f32 dot small bins", ip, ix, q, k, v, "f32", light_max_deg=4,
               hub_min_deg_exclusive=9, hub_chunk=3)


@pytest.mark.parametrize("tl,th,c", [(8, 64, 32), (16, 1024, 512), (0, 0, 5)])
def test_chunglu20k_bf16_forward_every_row(tl, th, c):
    w = gg.WORKLOADS["chunglu1m_dot_bf16"]
    ip, ix = gg.make_graph(w, n=20_000)
    q, k, v = gg.make_features(w, n=20_000)
    plan, *_ = fwd_parity("chunglu20k bf16 dot", ip, ix, q, k, v, "bf16", light_max_deg=tl,
                          hub_min_deg_exclusive=th, hub_chunk=c)
    info = plan.info()
    assert info["n_row_hub"] > 0 and info["n_row_chunks"] > info["n_row_hub"]


def test_gat_chunglu100k_f32_forward_every_row():
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    ip, ix = gg.make_graph(w)
    s, t, v = gg.make_features(w)
    plan, *_ = fwd_parity("chunglu100k f32 gat", ip, ix, s, t, v, "f32", score="gat",
                          scale=1.0, neg_slope=0.2)
    assert plan.info()["n_row_hub"] > 0


def test_gat_scale_and_slope_bf16():
    rng = np.random.default_rng(4)
    ip, ix = gg.random_multigraph(3000, 60000, rng, hub_rows=(7,), hub_deg=5000)
    s = rng.standard_normal((3000, 2)).astype(np.float32)
    t = rng.standard_normal((3000, 2)).astype(np.float32)
    v = gg.f32_to_bf16_bits(rng.standard_normal((3000, 2, 64)).astype(np.float32))
    fwd_parity("gat bf16 scale 1.7 slope 0.05", ip, ix, s, t, v, "bf16", score="gat",
               scale=1.7, neg_slope=0.05, light_max_deg=8, hub_min_deg_exclusive=32, hub_chunk=64)


def test_rmat16k_bf16_d128_forward_every_row():
    w = gg.WORKLOADS["rmat21_dot_bf16"]
    ip, ix = gg.make_graph(w, n=1 << 14)
    q, k, v = gg.make_features(w, n=1 << 14)
    fwd_parity("rmat 2^14 bf16 d128", ip, ix, q, k, v, "bf16", light_max_deg=8,
               hub_min_deg_exclusive=256, hub_chunk=128)


GEOMS = [(G, LH) for G in (4, 8, 16, 32, 64) for LH in (2, 4, 8, 16, 32, 64) if LH <= G]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_every_compiled_geometry(dtype, G, LH):
    eb = 4 if dtype == "f32" else 2
    H, d = G // LH, LH * 16 // eb
    rng = np.random.default_rng(G * 100 + LH)
    n = 400
    ip, ix = gg.random_multigraph(n, 3000, rng, hub_rows=(3,), hub_deg=700)
    feats = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    fwd_parity(f"geometry G{G} LH{LH}", ip, ix, *feats, dtype, light_max_deg=6,
               hub_min_deg_exclusive=20, hub_chunk=16)
    if G in (8, 64):
        s = rng.standard_normal((n, H)).astype(np.float32)
        t = rng.standard_normal((n, H)).astype(np.float32)
        fwd_parity(f"geometry G{G} LH{LH} gat", ip, ix, s, t, feats[2], dtype, score="gat",
                   light_max_deg=6, hub_min_deg_exclusive=20, hub_chunk=16)


def test_empty_rows_single_neighbours_and_parallel_edges():
    rng = np.random.default_rng(9)
    n, H, d = 500, 4, 32
    dst = np.r_[np.arange(100, 200),                   # rows 100..199: exactly one edge
                np.repeat(np.arange(200, 300), 5),     # 5 edges each
                np.full(40, 300), np.full(3000, 301)]  # a medium row and a hub row
    src = rng.integers(0, n, dst.size)
    src[np.flatnonzero(dst == 300)[:20]] = 17          # 20 parallel 17 -> 300 edges
    ip, ix = gg.csr_from_edges(n, src, dst)           # rows 0..99 and 302..499 are empty
    q, k, v = (gg.f32_to_bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
               for _ in range(3))
    plan, out, lse, _ = fwd_parity("empty/single/parallel", ip, ix, q, k, v, "bf16",
                                   light_max_deg=4, hub_min_deg_exclusive=64, hub_chunk=100)
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    empty = np.diff(ip) == 0
    assert np.all(o[empty] == 0)
    assert np.all(np.isneginf(lse.cpu().numpy()[empty]))
    single = np.flatnonzero(np.diff(ip) == 1)
    assert np.array_equal(o[single], v[ix[ip[single]]])   # bitwise: weight exactly 1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_star_hub_row_200k(dtype):
    """One destination with 200,000 in-edges (hundreds of chunks, ordered merge)."""
    rng = np.random.default_rng(11)
    n, H, d = 250_000, 2, 64
    src = rng.integers(0, n, 200_000)
    ip, ix = gg.csr_from_edges(n, np.r_[src, np.arange(n)], np.r_[np.zeros(200_000, np.int64),
                                                                  np.arange(n)])
    feats = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    rows = np.r_[0, rng.integers(1, n, 50)]
    plan, *_ = fwd_parity(f"star 200k {dtype}", ip, ix, *feats, dtype, rows=rows)
    assert plan.info()["max_in_degree"] == 200_001


# ------------------------------------------------------------------ backward

def bwd_case(tag, ip, ix, q, k, v, dout, dtype, rows=None, cols=None, **plan_kw):
    d = q.shape[2]
    scale = f32(1 / math.sqrt(d))
    say(tag, "N", ip.size - 1, "E", ix.size, "H", q.shape[1], "d", d, dtype, plan_kw)
    plan = Plan(ip, ix, **plan_kw).upload()
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(dout)
    out, lse = fwd(plan, tq, tk, tv, scale=scale)
    dq, dk, dv = bwd(plan, tq, tk, tv, tdo, lse, scale=scale)
    torch.cuda.synchronize()
    if rows is None:
        rq, rk, rv = A.backward(ip, ix, q, k, v, dout, scale)
        errs = [check(f"{tag} dq", host64(dq), rq, dtype),
                check(f"{tag} dk", host64(dk), rk, dtype),
                check(f"{tag} dv", host64(dv), rv, dtype)]
    else:
        rq = A.grad_q_rows(ip, ix, q, k, v, dout, rows, scale)
        rk, rv = A.grad_kv_cols(ip, ix, q, k, v, dout, cols, scale)
        rt, ct = torch.from_numpy(np.asarray(rows)).cuda(), torch.from_numpy(np.asarray(cols)).cuda()
        errs = [check(f"{tag} dq", host64(dq[rt]), rq, dtype),
                check(f"{tag} dk", host64(dk[ct]), rk, dtype),
                check(f"{tag} dv", host64(dv[ct]), rv, dtype)]
    say(tag, "max abs / norm-rel errors", errs)
    return plan, (out, lse, dq, dk, dv)


@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype,H,d", [("bf16", 8, 32), ("f32", 4, 32), ("bf16", 2, 128)])
def test_feature_slices_every_element(S, dtype, H, d):
    """Feature slices dealt to XCDs (forward and the dQ pass): every element against the
    oracle for each slice count, including forced counts that fall back for wide heads, and
    the same result twice in a row."""
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 3000
    ip, ix = gg.make_graph(w, n=n)
    rng = np.random.default_rng(31 + S)
    feats = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(4)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    plan, res = bwd_case(f"slices {S} {dtype} H{H} d{d}", ip, ix, *feats, dtype, light_max_deg=8,
                         hub_min_deg_exclusive=64, hub_chunk=32, feature_slices=S)
    assert plan.info()["feature_slices"] == S
    q, k, v, do = (dev(x) for x in feats)
    scale = f32(1 / math.sqrt(d))
    out, lse = fwd(plan, q, k, v, scale=scale)
    dq, dk, dv = bwd(plan, q, k, v, do, lse, scale=scale)
    for a, b in zip(res, (out, lse, dq, dk, dv)):
        assert torch.equal(a, b)
    ro, rl = A.forward(ip, ix, *feats[:3], "dot", scale)
    check(f"slices {S} out", host64(out), ro, dtype)
    check_lse(f"slices {S} lse", host64(lse), rl)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_chunglu5k_every_element(dtype):
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 5000
    ip, ix = gg.make_graph(w, n=n)
    rng = np.random.default_rng(21)
    feats = [rng.standard_normal((n, 8, 32)).astype(np.float32) for _ in range(4)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    plan, _ = bwd_case(f"bwd chunglu5k {dtype}", ip, ix, *feats, dtype, light_max_deg=8,
                       hub_min_deg_exclusive=64, hub_chunk=32)
    info = plan.info()
    assert info["n_col_hub"] > 0 and info["n_col_chunks"] > info["n_col_hub"]
    assert info["n_row_hub"] > 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_backward_geometries(G, LH, dtype):
    """The dot backward on every element, for every compiled (lanes per row, lanes per head)
    geometry, with a row hub and a column hub split into chunks."""
    eb = 4 if dtype == "f32" else 2
    H, d = G // LH, LH * 16 // eb
    rng = np.random.default_rng(G + LH)
    n = 300
    src = np.r_[rng.integers(0, n, 2500), np.full(600, 5)]       # column hub 5
    dst = np.r_[rng.integers(0, n, 2500), rng.integers(0, n, 600)]
    dst[:500] = 9                                               # row hub 9
    ip, ix = gg.csr_from_edges(n, src, dst)
    feats = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(4)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    bwd_case(f"bwd geometry G{G} LH{LH} {dtype}", ip, ix, *feats, dtype, light_max_deg=4,
             hub_min_deg_exclusive=40, hub_chunk=16)


def test_backward_empty_rows_and_star_column():
    rng = np.random.default_rng(31)
    n, H, d = 60_000, 2, 32
    src = np.r_[np.zeros(50_000, np.int64), rng.integers(0, n, 20_000)]   # node 0: source hub
    dst = np.r_[rng.integers(0, 30_000, 50_000), rng.integers(0, 30_000, 20_000)]
    ip, ix = gg.csr_from_edges(n, src, dst)          # rows >= 30000 are empty
    feats = [gg.f32_to_bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
             for _ in range(4)]
    rows = np.r_[rng.integers(0, 30_000, 100), rng.integers(30_000, n, 20)]
    cols = np.r_[0, rng.integers(1, n, 60)]
    plan, (out, lse, dq, dk, dv) = bwd_case("bwd star column", ip, ix, *feats, "bf16",
                                            rows=rows, cols=cols)
    assert plan.info()["max_out_degree"] >= 50_000
    empty = torch.from_numpy(np.flatnonzero(np.diff(ip) == 0)).cuda()
    assert torch.all(dq[empty] == 0)


def test_autograd_wrapper_matches_direct_calls():
    w = gg.WORKLOADS["chunglu1m_dot_bf16"]
    ip, ix = gg.make_graph(w, n=3000)
    q, k, v = gg.make_features(w, n=3000)
    say("autograd wrapper")
    plan = Plan(ip, ix).upload()
    tq, tk, tv = (dev(x).requires_grad_(True) for x in (q, k, v))
    out = graph_attention(plan, tq, tk, tv)
    g = torch.randn_like(out)
    out.backward(g)
    o2, lse = fwd(plan, tq.detach(), tk.detach(), tv.detach())
    d2 = bwd(plan, tq.detach(), tk.detach(), tv.detach(), g, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for a, b in zip((tq.grad, tk.grad, tv.grad), d2):
        assert torch.equal(a, b)


def test_autograd_wrappers_of_gat_and_gatv2():
    """The GAT-style and GATv2 autograd ops give the direct calls' outputs and gradients bit
    for bit, and a layer stacked on another (the gradient flows through both) matches the
    oracle chained by hand."""
    from sparse_graph_attention_02_amd import graph_attention_gatv2
    rng = np.random.default_rng(44)
    n, H, d = 2000, 4, 32
    ip, ix = gg.random_multigraph(n, 20_000, rng, hub_rows=(3,), hub_deg=1500)
    plan = Plan(ip, ix).upload()
    say("autograd wrappers: GAT-style and GATv2")
    s_, t_ = (torch.from_numpy(rng.standard_normal((n, H)).astype(np.float32)).cuda()
              .requires_grad_(True) for _ in range(2))
    v = torch.from_numpy(rng.standard_normal((n, H, d)).astype(np.float32)).cuda() \
        .requires_grad_(True)
    out = graph_attention(plan, s_, t_, v, score="gat", neg_slope=0.15)
    g = torch.randn_like(out)
    out.backward(g)
    o2, lse = fwd(plan, s_.detach(), t_.detach(), v.detach(), score="gat", neg_slope=0.15)
    d2 = bwd(plan, s_.detach(), t_.detach(), v.detach(), g, lse, score="gat", neg_slope=0.15)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for a, b in zip((s_.grad, t_.grad, v.grad), d2):
        assert torch.equal(a, b)
    # GATv2, fp32, with its attention vector trained too
    xd, xs = (torch.from_numpy(rng.standard_normal((n, H, d)).astype(np.float32)).cuda()
              .requires_grad_(True) for _ in range(2))
    attn = torch.from_numpy((rng.standard_normal((H, d)) / 6).astype(np.float32)).cuda() \
        .requires_grad_(True)
    out = graph_attention_gatv2(plan, xd, xs, attn, 0.9)
    g = torch.randn_like(out)
    out.backward(g)
    from sparse_graph_attention_02_amd import bwd_gatv2, fwd_gatv2
    o2, lse = fwd_gatv2(plan, xd.detach(), xs.detach(), attn.detach(), scale=0.9)
    d2 = bwd_gatv2(plan, xd.detach(), xs.detach(), attn.detach(), g, lse, scale=0.9)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for a, b in zip((xd.grad, xs.grad, attn.grad), d2):
        assert torch.equal(a, b)
    # two stacked layers (the second's queries are the first's output), against the oracle
    # chained by hand: forward through both, backward through both
    q0, k0, v0, k1, v1 = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(5))
    tq0, tk0, tv0, tk1, tv1 = (torch.from_numpy(x).cuda().requires_grad_(True)
                               for x in (q0, k0, v0, k1, v1))
    h = graph_attention(plan, tq0, tk0, tv0)
    y = graph_attention(plan, h, tk1, tv1)
    gy = rng.standard_normal((n, H, d)).astype(np.float32)
    y.backward(torch.from_numpy(gy).cuda())
    torch.cuda.synchronize()
    sc = f32(1 / math.sqrt(d))
    rh, _ = A.forward(ip, ix, q0, k0, v0, "dot", sc)
    h32 = host64(h).astype(np.float32)                  # the stored activation
    dq1, dk1, dv1 = A.backward(ip, ix, h32, k1, v1, gy, sc)
    dq0, dk0, dv0 = A.backward(ip, ix, q0, k0, v0, dq1.astype(np.float32), sc)
    check("stacked h", host64(h), rh, "f32")
    for name, gt, ref in (("dk1", tk1, dk1), ("dv1", tv1, dv1), ("dq0", tq0, dq0),
                          ("dk0", tk0, dk0), ("dv0", tv0, dv0)):
        check(f"stacked {name}", host64(gt.grad), ref, "f32")


# ------------------------------------------------------------------ determinism, memory

def test_bitwise_deterministic_fwd_bwd():
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    ip, ix = gg.make_graph(w, n=50_000)
    q, k, v = gg.make_features(w, n=50_000)
    dout = gg.make_dout(w, n=50_000)
    say("determinism chunglu50k")
    plan = Plan(ip, ix, light_max_deg=8, hub_min_deg_exclusive=128, hub_chunk=64).upload()
    tq, tk, tv, td = dev(q), dev(k), dev(v), dev(dout)
    res = []
    for _ in range(2):
        out, lse = fwd(plan, tq, tk, tv)
        res.append((out, lse) + bwd(plan, tq, tk, tv, td, lse))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_no_edge_sized_allocation():
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 200_000
    ip, ix = gg.make_graph(w, n=n)
    q, k, v = gg.make_features(w, n=n)
    dout = gg.make_dout(w, n=n)
    say("memory chunglu200k E", ix.size)
    plan = Plan(ip, ix).upload()
    tq, tk, tv, td = dev(q), dev(k), dev(v), dev(dout)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    out, lse = fwd(plan, tq, tk, tv)
    dq, dk, dv = bwd(plan, tq, tk, tv, td, lse)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    feat = tq.numel() * tq.element_size()
    ws = plan.fwd_workspace_bytes(8, 32) + plan.bwd_workspace_bytes(8, 32)
    expected = 4 * feat + lse.numel() * 4 + ws       # out, dq, dk, dv + lse + workspaces
    e_scores = ix.size * 8 * 4                         # an E x H fp32 score tensor
    say("peak delta", peak, "expected", expected, "E*H*4", e_scores)
    assert peak <= expected + (4 << 20)
    assert ws < e_scores / 4


# ------------------------------------------------------------------ full workload sizes

# Plans of the full-size tests: the library default, and the XCD split bench.py uses for
# the dot-score workloads (rows above 256 and columns above 1024 edges regrouped, columns
# in 1024-edge chunks)
FULL_PLANS = [pytest.param({}, id="default-plan"),
              pytest.param(dict(xcd_split_min_deg_exclusive=256,
                                col_xcd_split_min_deg_exclusive=1024, col_hub_chunk=1024),
                           id="bench-split-plan")]


def test_full_plans_match_the_bench():
    import bench
    for name in ("chunglu1m_train_bf16", "chunglu1m_dot_bf16", "rmat21_dot_bf16"):
        assert FULL_PLANS[1].values[0] == bench.bench_plan_kw(gg.WORKLOADS[name])


# The 1M training step (and so the 1M forward) and the R-MAT forward are checked on every
# element in the bench's split plan by tests/test_gpu_fullsize.py; on the default plan
# their full-size checks below sample rows and columns.
def _sample_rows(ip, rng, k=256):
    deg = np.diff(ip)
    top = np.argsort(-deg, kind="stable")[:8]
    ones = np.flatnonzero(deg == 1)[:8]
    return np.unique(np.r_[top, ones, rng.choice(ip.size - 1, k, replace=False)])


@pytest.mark.slow
@pytest.mark.parametrize("plan_kw", FULL_PLANS[:1])
def test_full_chunglu1m_bf16_forward_sampled(plan_kw):
    w = gg.WORKLOADS["chunglu1m_dot_bf16"]
    ip, ix = gg.make_graph(w)
    q, k, v = gg.make_features(w)
    rows = _sample_rows(ip, np.random.default_rng(3))
    fwd_parity("full chunglu1m bf16 dot (sampled rows)", ip, ix, q, k, v, "bf16", rows=rows,
               build_csc=False, **plan_kw)


@pytest.mark.slow
@pytest.mark.parametrize("plan_kw", FULL_PLANS[:1])
def test_full_rmat21_bf16_forward_sampled(plan_kw):
    w = gg.WORKLOADS["rmat21_dot_bf16"]
    ip, ix = gg.make_graph(w)
    q, k, v = gg.make_features(w)
    rows = _sample_rows(ip, np.random.default_rng(4))
    plan, *_ = fwd_parity("full rmat21 bf16 dot (sampled rows)", ip, ix, q, k, v, "bf16",
                          rows=rows, build_csc=False, **plan_kw)
    assert plan.info()["max_in_degree"] > 100_000


@pytest.mark.slow
@pytest.mark.parametrize("plan_kw", FULL_PLANS)
def test_full_chunglu100k_gat_f32_forward_sampled(plan_kw):
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    ip, ix = gg.make_graph(w)
    s, t, v = gg.make_features(w)
    rows = _sample_rows(ip, np.random.default_rng(5), k=2000)
    fwd_parity("full chunglu100k gat (sampled rows)", ip, ix, s, t, v, "f32", score="gat",
               scale=1.0, rows=rows, build_csc=False, **plan_kw)


@pytest.mark.slow
@pytest.mark.parametrize("plan_kw", FULL_PLANS[:1])
def test_full_chunglu1m_training_step_sampled(plan_kw):
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    ip, ix = gg.make_graph(w)
    q, k, v = gg.make_features(w)
    dout = gg.make_dout(w)
    rng = np.random.default_rng(6)
    rows = _sample_rows(ip, rng, k=128)
    odeg = np.bincount(ix, minlength=w.n)
    cols = np.unique(np.r_[np.argsort(-odeg, kind="stable")[:3],
                           np.flatnonzero(odeg == 1)[:4], rng.choice(w.n, 48, replace=False)])
    plan, r = bwd_case("full chunglu1m training step (sampled rows/cols)", ip, ix, q, k, v,
                       dout, "bf16", rows=rows, cols=cols, **plan_kw)
    ro, rl = A.forward_rows(ip, ix, q, k, v, rows, "dot", f32(1 / math.sqrt(w.dim)))
    rt = torch.from_numpy(rows).cuda()
    check("full chunglu1m training step out", host64(r[0][rt]), ro, "bf16")
    check_lse("full chunglu1m training step lse", host64(r[1][rt]), rl)


@pytest.mark.parametrize("plan_kw", FULL_PLANS)
def test_gather_probes_run_on_the_plan_graph(plan_kw):
    """The probes run over the plan's own work lists (rows and, with the transpose,
    columns) and the random-table probe over a table; none writes its sink."""
    w = gg.WORKLOADS["chunglu1m_dot_bf16"]
    ip, ix = gg.make_graph(w, n=20_000)
    q, k, v = gg.make_features(w, n=20_000)
    say("gather probes chunglu20k", plan_kw)
    from sparse_graph_attention_02_amd import gather_probe, gather_probe_cols, gather_probe_random
    plan = Plan(ip, ix, **plan_kw).upload()
    tq, tk, tv = dev(q), dev(k), dev(v)
    rec = torch.zeros((20_000, 8, 2), dtype=torch.float32, device="cuda")
    sinks = [gather_probe(plan, tk, tv, row_a=tq),
             gather_probe(plan, tk, row_a=tq, row_b=tv),
             gather_probe_cols(plan, tv, q=tq, record=rec, k=tk, v=tv),
             gather_probe_cols(plan, tv),
             gather_probe_random(tk, 512, 100_000),
             gather_probe_random(tk, 64, 1000, table_rows=7)]
    torch.cuda.synchronize()
    for s in sinks:   # a probe writes its sink only on a 96-bit XOR collision
        assert int(s.sum()) == 0


# ------------------------------------------------------------------ GAT-style backward

def gat_bwd_case(tag, ip, ix, s, t, v, dout, dtype, scale=1.0, slope=0.2, rows=None, cols=None,
                 **plan_kw):
    say(tag, "N", ip.size - 1, "E", ix.size, "H", v.shape[1], "d", v.shape[2], dtype, plan_kw)
    plan = Plan(ip, ix, **plan_kw).upload()
    ts, tt, tv, td = dev(s), dev(t), dev(v), dev(dout)
    out, lse = fwd(plan, ts, tt, tv, score="gat", scale=scale, neg_slope=slope)
    ds, dt, dv = bwd(plan, ts, tt, tv, td, lse, score="gat", scale=scale, neg_slope=slope)
    torch.cuda.synchronize()
    if rows is None:
        rs, rt, rv = A.backward_gat(ip, ix, s, t, v, dout, scale, f32(slope))
        errs = [check(f"{tag} ds", host64(ds), rs, dtype), check(f"{tag} dt", host64(dt), rt, dtype),
                check(f"{tag} dv", host64(dv), rv, dtype)]
    else:
        rs = A.grad_s_rows(ip, ix, s, t, v, dout, rows, scale, f32(slope))
        rt, rv = A.grad_tv_cols(ip, ix, s, t, v, dout, cols, scale, f32(slope))
        r_t, c_t = torch.from_numpy(np.asarray(rows)).cuda(), torch.from_numpy(np.asarray(cols)).cuda()
        errs = [check(f"{tag} ds", host64(ds[r_t]), rs, dtype),
                check(f"{tag} dt", host64(dt[c_t]), rt, dtype),
                check(f"{tag} dv", host64(dv[c_t]), rv, dtype)]
    say(tag, "max abs / norm-rel errors", errs)
    return plan, (ds, dt, dv)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gat_backward_every_element(dtype):
    rng = np.random.default_rng(41)
    n, H, d = 3000, 4, 64
    src = np.r_[rng.integers(0, n, 40_000), np.full(3000, 11)]      # column hub 11
    dst = np.r_[rng.integers(0, n, 40_000), rng.integers(0, n, 3000)]
    dst[:4000] = 7                                                  # row hub 7
    ip, ix = gg.csr_from_edges(n, src, dst)
    s = rng.standard_normal((n, H)).astype(np.float32)
    t = rng.standard_normal((n, H)).astype(np.float32)
    v, do = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(2))
    if dtype == "bf16":
        v, do = gg.f32_to_bf16_bits(v), gg.f32_to_bf16_bits(do)
    plan, _ = gat_bwd_case(f"gat bwd {dtype}", ip, ix, s, t, v, do, dtype, scale=1.3, slope=0.1,
                           light_max_deg=8, hub_min_deg_exclusive=64, hub_chunk=100)
    info = plan.info()
    assert info["n_row_chunks"] > info["n_row_hub"] > 0
    assert info["n_col_chunks"] > info["n_col_hub"] > 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_gat_backward_geometries(G, LH, dtype):
    """The GAT-style backward on every element, for every compiled geometry of V."""
    eb = 4 if dtype == "f32" else 2
    H, d = G // LH, LH * 16 // eb
    rng = np.random.default_rng(G * 7 + LH)
    n = 400
    ip, ix = gg.random_multigraph(n, 4000, rng, hub_rows=(3,), hub_deg=500)
    s, t = (rng.standard_normal((n, H)).astype(np.float32) for _ in range(2))
    v, do = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(2))
    if dtype == "bf16":
        v, do = gg.f32_to_bf16_bits(v), gg.f32_to_bf16_bits(do)
    gat_bwd_case(f"gat bwd geometry G{G} LH{LH} {dtype}", ip, ix, s, t, v, do, dtype,
                 light_max_deg=4, hub_min_deg_exclusive=30, hub_chunk=16)


def test_gat_backward_deterministic():
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    ip, ix = gg.make_graph(w, n=20_000)
    s, t, v = gg.make_features(w, n=20_000)
    do = np.random.default_rng(3).standard_normal(v.shape).astype(np.float32)
    say("gat bwd determinism")
    plan = Plan(ip, ix, light_max_deg=8, hub_min_deg_exclusive=128, hub_chunk=64).upload()
    ts, tt, tv, td = dev(s), dev(t), dev(v), dev(do)
    res = []
    for _ in range(2):
        out, lse = fwd(plan, ts, tt, tv, score="gat")
        res.append(bwd(plan, ts, tt, tv, td, lse, score="gat"))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.slow
@pytest.mark.parametrize("plan_kw", FULL_PLANS)
def test_full_chunglu100k_gat_backward_sampled(plan_kw):
    """The GAT training step as the bench runs it (same graph, features, dOut; the default
    and the bench's split plan): ds on sampled rows, dt and dV on sampled columns including
    the top hubs."""
    w = gg.WORKLOADS["chunglu100k_gat_train_f32"]
    ip, ix = gg.make_graph(w)
    s, t, v = gg.make_features(w)
    do = gg.make_dout(w)
    rng = np.random.default_rng(8)
    rows = _sample_rows(ip, rng, k=500)
    odeg = np.bincount(ix, minlength=w.n)
    cols = np.unique(np.r_[np.argsort(-odeg, kind="stable")[:3], rng.choice(w.n, 200, replace=False)])
    gat_bwd_case("full chunglu100k gat bwd (sampled)", ip, ix, s, t, v, do, "f32", rows=rows,
                 cols=cols, **plan_kw)


# ------------------------------------------------------------------ GATv2

def gatv2_fwd_case(tag, ip, ix, xd, xs, a, dtype, scale=1.0, slope=0.2, rows=None, **plan_kw):
    from sparse_graph_attention_02_amd import fwd_gatv2
    say(tag, "N", ip.size - 1, "E", ix.size, "H", xs.shape[1], "d", xs.shape[2], dtype, plan_kw)
    plan = Plan(ip, ix, **plan_kw).upload()
    out, lse = fwd_gatv2(plan, dev(xd), dev(xs), dev(a), scale=scale, neg_slope=slope)
    torch.cuda.synchronize()
    rows = np.arange(ip.size - 1) if rows is None else np.asarray(rows)
    ro, rl = A.forward_gatv2_rows(ip, ix, xd, xs, a, rows, scale, f32(slope))
    rt = torch.from_numpy(rows).cuda()
    check(f"{tag} out", host64(out[rt]), ro, dtype)
    check_lse(f"{tag} lse", host64(lse[rt]), rl)
    return plan, out, lse


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_gatv2_forward_geometries(dtype, G, LH):
    eb = 4 if dtype == "f32" else 2
    H, d = G // LH, LH * 16 // eb
    rng = np.random.default_rng(G * 13 + LH)
    n = 500
    ip, ix = gg.random_multigraph(n, 5000, rng, hub_rows=(2,), hub_deg=900)
    xd, xs = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(2))
    a = (rng.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        xd, xs = gg.f32_to_bf16_bits(xd), gg.f32_to_bf16_bits(xs)
    gatv2_fwd_case(f"gatv2 fwd G{G} LH{LH} {dtype}", ip, ix, xd, xs, a, dtype, scale=1.2,
                   slope=0.2, light_max_deg=6, hub_min_deg_exclusive=24, hub_chunk=16)


@pytest.mark.parametrize("dtype,H,d", [("bf16", 8, 32), ("f32", 4, 32), ("bf16", 2, 64)])
def test_gatv2_forward_feature_slices(dtype, H, d):
    """An explicit feature-slice count in the GATv2 forward: every element against the
    oracle for each count, and the same bits again on a second call. (Counts differ in how
    a row's edges are dealt to lane groups, so they differ from one another in rounding.)"""
    rng = np.random.default_rng(H * 7 + d)
    n = 1500
    ip, ix = gg.random_multigraph(n, 15000, rng, hub_rows=(4, 9), hub_deg=700)
    xd, xs = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(2))
    a = (rng.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        xd, xs = gg.f32_to_bf16_bits(xd), gg.f32_to_bf16_bits(xs)
    from sparse_graph_attention_02_amd import fwd_gatv2
    kw = dict(light_max_deg=8, hub_min_deg_exclusive=64, hub_chunk=48)
    for S in (1, 2, 4, 8):
        plan, out, lse = gatv2_fwd_case(f"gatv2 slices {S} {dtype}", ip, ix, xd, xs, a, dtype,
                                        feature_slices=S, **kw)
        assert plan.info()["feature_slices"] == S
        out2, lse2 = fwd_gatv2(plan, dev(xd), dev(xs), dev(a))
        assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_gatv2_forward_chunglu100k_every_row():
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    ip, ix = gg.make_graph(w)
    rng = np.random.default_rng(17)
    xd, xs = (rng.standard_normal((w.n, 4, 64)).astype(np.float32) for _ in range(2))
    a = (rng.standard_normal((4, 64)) / 8).astype(np.float32)
    plan, out, lse = gatv2_fwd_case("gatv2 chunglu100k f32", ip, ix, xd, xs, a, "f32")
    assert plan.info()["n_row_hub"] > 0


def gatv2_bwd_case(tag, ip, ix, xd, xs, a, do, dtype, scale=1.0, slope=0.2, rows=None, cols=None,
                   **plan_kw):
    from sparse_graph_attention_02_amd import bwd_gatv2, fwd_gatv2
    say(tag, "N", ip.size - 1, "E", ix.size, "H", xs.shape[1], "d", xs.shape[2], dtype, plan_kw)
    plan = Plan(ip, ix, **plan_kw).upload()
    txd, txs, ta, td = dev(xd), dev(xs), dev(a), dev(do)
    out, lse = fwd_gatv2(plan, txd, txs, ta, scale=scale, neg_slope=slope)
    dxd, dxs, da = bwd_gatv2(plan, txd, txs, ta, td, lse, scale=scale, neg_slope=slope)
    torch.cuda.synchronize()
    sl = f32(slope)
    if rows is None:
        rxd, rxs, rda = A.backward_gatv2(ip, ix, xd, xs, a, do, scale, sl)
        errs = [check(f"{tag} dxd", host64(dxd), rxd, dtype), check(f"{tag} dxs", host64(dxs), rxs, dtype)]
    else:
        rxd, _ = A.grad_gatv2_rows(ip, ix, xd, xs, a, do, rows, scale, sl)
        rxs = A.grad_gatv2_cols(ip, ix, xd, xs, a, do, cols, scale, sl)
        r_t, c_t = torch.from_numpy(np.asarray(rows)).cuda(), torch.from_numpy(np.asarray(cols)).cuda()
        errs = [check(f"{tag} dxd", host64(dxd[r_t]), rxd, dtype),
                check(f"{tag} dxs", host64(dxs[c_t]), rxs, dtype)]
        _, rda = A.grad_gatv2_rows(ip, ix, xd, xs, a, do, np.arange(ip.size - 1), scale, sl)
    errs.append(check(f"{tag} dattn", host64(da), rda, dtype))
    say(tag, "max abs / norm-rel errors", errs)
    return plan, (dxd, dxs, da)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_gatv2_backward_every_element(dtype, G, LH):
    eb = 4 if dtype == "f32" else 2
    H, d = G // LH, LH * 16 // eb
    rng = np.random.default_rng(G * 31 + LH)
    n = 600
    src = np.r_[rng.integers(0, n, 6000), np.full(900, 13)]       # column hub 13
    dst = np.r_[rng.integers(0, n, 6000), rng.integers(0, n, 900)]
    dst[:800] = 5                                                 # row hub 5
    ip, ix = gg.csr_from_edges(n, src, dst)
    xd, xs, do = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(3))
    a = (rng.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        xd, xs, do = (gg.f32_to_bf16_bits(x) for x in (xd, xs, do))
    plan, _ = gatv2_bwd_case(f"gatv2 bwd G{G} LH{LH} {dtype}", ip, ix, xd, xs, a, do, dtype,
                             scale=1.1, slope=0.2, light_max_deg=6, hub_min_deg_exclusive=40,
                             hub_chunk=32)
    info = plan.info()
    assert info["n_row_chunks"] > info["n_row_hub"] > 0 and info["n_col_chunks"] > info["n_col_hub"] > 0


def test_gatv2_backward_deterministic_and_empty_graph():
    from sparse_graph_attention_02_amd import bwd_gatv2, fwd_gatv2
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    ip, ix = gg.make_graph(w, n=20_000)
    rng = np.random.default_rng(5)
    xd, xs, do = (gg.f32_to_bf16_bits(rng.standard_normal((20_000, 4, 64)).astype(np.float32))
                  for _ in range(3))
    a = (rng.standard_normal((4, 64)) / 8).astype(np.float32)
    say("gatv2 determinism")
    plan = Plan(ip, ix, light_max_deg=8, hub_min_deg_exclusive=128, hub_chunk=64).upload()
    t = [dev(x) for x in (xd, xs, a, do)]
    res = []
    for _ in range(2):
        out, lse = fwd_gatv2(plan, t[0], t[1], t[2])
        res.append((out, lse) + bwd_gatv2(plan, t[0], t[1], t[2], t[3], lse))
    torch.cuda.synchronize()
    for x, y in zip(*res):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    # a graph with no nodes: dattn comes back as zeros
    empty = Plan(np.zeros(1, np.int32), np.zeros(0, np.int32)).upload()
    z = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    dattn = torch.full((4, 64), 7.0, device="cuda")
    bwd_gatv2(empty, z, z, t[2], z, torch.zeros((0, 4), device="cuda"), dattn=dattn)
    torch.cuda.synchronize()
    assert torch.all(dattn == 0)


@pytest.mark.slow
def test_full_chunglu100k_gatv2_backward_sampled():
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    ip, ix = gg.make_graph(w)
    rng = np.random.default_rng(9)
    xd, xs, do = (rng.standard_normal((w.n, 4, 64)).astype(np.float32) for _ in range(3))
    a = (rng.standard_normal((4, 64)) / 8).astype(np.float32)
    rows = _sample_rows(ip, rng, k=300)
    odeg = np.bincount(ix, minlength=w.n)
    cols = np.unique(np.r_[np.argsort(-odeg, kind="stable")[:2], rng.choice(w.n, 100, replace=False)])
    gatv2_bwd_case("full chunglu100k gatv2 bwd (sampled)", ip, ix, xd, xs, a, do, "f32", rows=rows,
                   cols=cols)


@pytest.mark.slow
@pytest.mark.parametrize("plan_kw", FULL_PLANS)
def test_full_chunglu1m_gatv2_training_step_sampled(plan_kw):
    """The GATv2 training step at full size (the default plan and the bench's split plan):
    forward and dxd on sampled rows (top hubs, single-neighbour rows, random rows),
    dxs on sampled columns, against the oracle; dattn, a sum over all 51M edges that the
    oracle cannot form here, by linearity: doubling dout doubles every gradient exactly."""
    from sparse_graph_attention_02_amd import bwd_gatv2, fwd_gatv2
    w = gg.WORKLOADS["chunglu1m_gatv2_train_bf16"]
    ip, ix = gg.make_graph(w)
    xd, xs, a = gg.make_features(w)
    do = gg.make_dout(w)
    say("full chunglu1m gatv2 training step (sampled)", "E", ix.size, plan_kw)
    plan = Plan(ip, ix, **plan_kw).upload()
    txd, txs, ta, td = dev(xd), dev(xs), dev(a), dev(do)
    out, lse = fwd_gatv2(plan, txd, txs, ta)
    dxd, dxs, da = bwd_gatv2(plan, txd, txs, ta, td, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = _sample_rows(ip, rng, k=48)
    odeg = np.bincount(ix, minlength=w.n)
    mid = np.flatnonzero((odeg > 100) & (odeg <= 400))
    cols = np.unique(np.r_[rng.choice(mid, 3, replace=False),
                           rng.choice(np.flatnonzero(odeg <= 16), 12, replace=False)])
    sl = f32(0.2)
    ro, rl = A.forward_gatv2_rows(ip, ix, xd, xs, a, rows, 1.0, sl)
    rt, ct = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    check("gatv2 1M out", host64(out[rt]), ro, "bf16")
    check_lse("gatv2 1M lse", host64(lse[rt]), rl)
    rxd, _ = A.grad_gatv2_rows(ip, ix, xd, xs, a, do, rows, 1.0, sl)
    check("gatv2 1M dxd", host64(dxd[rt]), rxd, "bf16")
    rxs = A.grad_gatv2_cols(ip, ix, xd, xs, a, do, cols, 1.0, sl)
    check("gatv2 1M dxs", host64(dxs[ct]), rxs, "bf16")
    assert torch.isfinite(da).all() and da.abs().sum() > 0
    dxd2, dxs2, da2 = bwd_gatv2(plan, txd, txs, ta, (td.float() * 2).to(td.dtype), lse)
    torch.cuda.synchronize()
    assert torch.equal(da2, da * 2)
    assert torch.equal(dxd2, dxd * 2) and torch.equal(dxs2, dxs * 2)


def test_binding_rejects_mismatched_rows():
    """The C calls take pointers only; the binding refuses tensors whose row count is not
    the plan's node count (the kernels would index past them)."""
    from sparse_graph_attention_02_amd import bwd_gatv2, fwd_gatv2, gather_probe
    say("binding row checks")
    ip, ix = gg.csr_from_edges(10, np.arange(10), (np.arange(10) + 1) % 10)
    plan = Plan(ip, ix).upload()
    x = torch.zeros((9, 2, 32), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((9, 2), device="cuda")
    attn = torch.zeros((2, 32), device="cuda")
    for call in (lambda: fwd(plan, x, x, x), lambda: bwd(plan, x, x, x, x, lse),
                 lambda: fwd_gatv2(plan, x, x, attn),
                 lambda: bwd_gatv2(plan, x, x, attn, x, lse),
                 lambda: gather_probe(plan, x, x)):
        with pytest.raises(ValueError):
            call()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_edge_chunks_in_every_layer(dtype):
    """Thresholds (0, 0, 1): every non-empty row and column is a hub cut into one-edge
    chunks, so each result comes out of the merge kernels alone. Dot, GAT-style and GATv2
    forward and backward, every element, against the oracle."""
    from sparse_graph_attention_02_amd import bwd_gatv2, fwd_gatv2
    rng = np.random.default_rng(61)
    n, H, d = 150, 2, 32 if dtype == "bf16" else 16
    ip, ix = gg.random_multigraph(n, 1200, rng, hub_rows=(4,), hub_deg=300)
    kw = dict(light_max_deg=0, hub_min_deg_exclusive=0, hub_chunk=1)
    feats = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(4)]
    if dtype == "bf16":
        feats = [gg.f32_to_bf16_bits(x) for x in feats]
    plan, _ = bwd_case(f"one-edge chunks dot {dtype}", ip, ix, *feats, dtype, **kw)
    info = plan.info()
    assert info["n_row_chunks"] == ix.size and info["n_col_chunks"] == ix.size
    s_, t_ = (rng.standard_normal((n, H)).astype(np.float32) for _ in range(2))
    gat_bwd_case(f"one-edge chunks gat {dtype}", ip, ix, s_, t_, feats[2], feats[3], dtype, **kw)
    a = (rng.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    gatv2_bwd_case(f"one-edge chunks gatv2 {dtype}", ip, ix, feats[0], feats[1], a, feats[3],
                   dtype, **kw)


@pytest.mark.parametrize("slope,scale", [(1.7, 0.6), (-0.3, 2.0), (0.0, 1.0)])
def test_gat_and_gatv2_slopes_and_scales(slope, scale):
    """LeakyReLU slopes above 1, negative and zero, and scales away from 1: the GAT-style and
    GATv2 layers, forward and backward on every element (the per-node form of the GATv2
    attention gradient relies on LeakyReLU(z) = g z, which holds for any slope)."""
    rng = np.random.default_rng(int(slope * 10) + 100)
    n, H, d = 300, 2, 16
    ip, ix = gg.random_multigraph(n, 3000, rng, hub_rows=(2,), hub_deg=400)
    kw = dict(light_max_deg=4, hub_min_deg_exclusive=48, hub_chunk=40)
    s_, t_ = (rng.standard_normal((n, H)).astype(np.float32) for _ in range(2))
    v, do = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(2))
    gat_bwd_case(f"gat slope {slope} scale {scale}", ip, ix, s_, t_, v, do, "f32", scale=scale,
                 slope=slope, **kw)
    xd, xs = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(2))
    a = (rng.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    gatv2_fwd_case(f"gatv2 slope {slope} scale {scale}", ip, ix, xd, xs, a, "f32", scale=scale,
                   slope=slope, **kw)
    gatv2_bwd_case(f"gatv2 slope {slope} scale {scale}", ip, ix, xd, xs, a, do, "f32",
                   scale=scale, slope=slope, **kw)
