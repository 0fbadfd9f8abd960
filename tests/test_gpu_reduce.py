"""GPU parity of the min / max neighbourhood reduction: the HIP path (through the C ABI)
against the fp64 oracle on the same seeded inputs.

The forward is index and selection work, so out and arg must be bit-exact (out bit
patterns included, which covers the sign of zero and infinities).  The backward sums
gradients, so dx is held to the float criteria of tests/gpu_util.py.  Every test prints
the case it is about to run.
"""
import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import planner as P
from oracle import reduction as R
from sparse_graph_attention_02_amd import (Plan, graph_reduce, reduce_bwd, reduce_fwd,
                                           reduce_slot_dtype)
from tests.gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def say(*a):
    print("[case]", *a, flush=True)


def bits(t):
    """Raw bit patterns of a GPU tensor (bf16 -> int16, fp32 -> int32)."""
    t = t.detach().cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def oracle_bits(vals, dtype):
    v32 = np.asarray(vals, np.float64).astype(np.float32)
    if dtype == "bf16":
        return gg.f32_to_bf16_bits(v32).view(np.int16)   # exact: values are bf16 already
    return v32.view(np.int32)


def slot_values(slot):
    """GPU slot tensor -> int64 row positions (all-ones -> -1)."""
    s = slot.cpu().numpy()
    if s.dtype == np.int16:
        v = s.view(np.uint16).astype(np.int64)
        return np.where(v == 0xFFFF, -1, v)
    v = s.view(np.uint32).astype(np.int64)
    return np.where(v == 0xFFFFFFFF, -1, v)


def fwd_exact(tag, ip, ix, x, dtype, op, rows=None, **plan_kw):
    say(tag, op, "N", ip.size - 1, "E", ix.size, "shape", x.shape, dtype, plan_kw)
    plan = Plan(ip, ix, **plan_kw).upload()
    out, arg, slot = reduce_fwd(plan, dev(x), op=op)
    torch.cuda.synchronize()
    rows = np.arange(ip.size - 1) if rows is None else np.asarray(rows)
    ro, ra = R.reduce_rows(ip, ix, x, rows, op)
    rt = torch.from_numpy(rows).cuda()
    F = ra.shape[1]
    ga = arg[rt].reshape(len(rows), F).cpu().numpy()
    bad = ga != ra
    assert not bad.any(), f"{tag}: {bad.sum()} args differ; first at " \
                          f"{np.argwhere(bad)[0]}: got {ga[bad][0]} ref {ra[bad][0]}"
    gb = bits(out[rt].reshape(len(rows), F))
    assert np.array_equal(gb, oracle_bits(ro, dtype)), f"{tag}: out bits differ"
    gs = slot_values(slot[rt].reshape(len(rows), F))
    # slots are positions in the plan's CSR (regrouped on XCD-split plans)
    pix = plan.array("indices")
    assert np.array_equal(np.sort(pix), np.sort(ix)) and (
        plan.info()["n_row_sched"] > 0 or np.array_equal(pix, ix))
    assert np.array_equal(gs, R.slots_of(ip, pix, rows, ra)), f"{tag}: slots differ"
    return plan, out, (arg, slot), ra


def bwd_parity(tag, plan, ip, ix, arg_slot, ref_arg, dout, dtype):
    """The GPU backward on the GPU forward's slot, and on its arg; the oracle backward on
    its own arg (the forward outputs were just shown to be identical).  Both GPU modes
    must agree bit for bit (same terms, same order)."""
    arg, slot = arg_slot
    say(tag, "backward", "N", ip.size - 1, "E", ix.size, dtype)
    td = dev(dout)
    dx = reduce_bwd(plan, None, td, slot=slot)
    dx_arg = reduce_bwd(plan, arg, td)
    torch.cuda.synchronize()
    ref = R.reduce_backward(ref_arg, dout, ip.size - 1)
    assert torch.equal(dx, dx_arg), f"{tag}: slot and arg backward differ"
    return dx, check(f"{tag} dx", host64(dx).reshape(ref.shape), ref, dtype)


SMALL_BINS = dict(light_max_deg=4, hub_min_deg_exclusive=9, hub_chunk=3)
SPLIT_BINS = dict(light_max_deg=4, hub_min_deg_exclusive=64, hub_chunk=5,
                  xcd_split_min_deg_exclusive=8)


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("bins", [{}, SMALL_BINS, SPLIT_BINS])
def test_er2k_f32_every_row(op, bins):
    w = gg.WORKLOADS["er2k_dot_f32"]
    ip, ix = gg.make_graph(w)
    x = gg.make_features(w)[0]                     # [2000, 1, 32] fp32: 128-byte rows
    plan, out, arg, ra = fwd_exact("er2k f32", ip, ix, x, "f32", op, **bins)
    dout = gg.make_features(w)[2]
    bwd_parity("er2k f32", plan, ip, ix, arg, ra, dout, "f32")


@pytest.mark.parametrize("tl,th,c", [(8, 64, 32), (16, 1024, 512), (0, 0, 5)])
def test_chunglu20k_bf16_every_row_and_backward(tl, th, c):
    w = gg.WORKLOADS["chunglu1m_max_train_bf16"]
    ip, ix = gg.make_graph(w, n=20_000)
    (x,) = gg.make_features(w, n=20_000)
    dout = gg.make_dout(w, n=20_000)
    for op in ("max", "min"):
        plan, out, arg, ra = fwd_exact("chunglu20k bf16", ip, ix, x, "bf16", op,
                                       light_max_deg=tl, hub_min_deg_exclusive=th, hub_chunk=c)
        info = plan.info()
        assert info["n_row_hub"] > 0 and info["n_col_hub"] > 0
        bwd_parity(f"chunglu20k bf16 {op}", plan, ip, ix, arg, ra, dout, "bf16")


@pytest.mark.parametrize("xs,cxs", [(16, 16), (40, 0), (0, 24)])
def test_chunglu20k_split_plans(xs, cxs):
    """Forward and backward on every row and element of a plan whose long rows and / or
    columns are regrouped by XCD: out and arg bit-exact, slots as positions in the plan's
    CSR, dx to the float criteria."""
    w = gg.WORKLOADS["chunglu1m_max_train_bf16"]
    ip, ix = gg.make_graph(w, n=20_000)
    (x,) = gg.make_features(w, n=20_000)
    dout = gg.make_dout(w, n=20_000)
    for op in ("max", "min"):
        plan, out, arg, ra = fwd_exact(f"chunglu20k split {xs}/{cxs}", ip, ix, x, "bf16", op,
                                       light_max_deg=8, hub_min_deg_exclusive=512, hub_chunk=16,
                                       xcd_split_min_deg_exclusive=xs,
                                       col_xcd_split_min_deg_exclusive=cxs)
        info = plan.info()
        assert (info["n_row_sched"] > 0) == (xs > 0) and (info["n_col_sched"] > 0) == (cxs > 0)
        bwd_parity(f"chunglu20k split {xs}/{cxs} {op}", plan, ip, ix, arg, ra, dout, "bf16")


@pytest.mark.parametrize("dtype,F", [("f32", 16), ("f32", 32), ("f32", 64), ("f32", 128),
                                     ("f32", 256), ("bf16", 32), ("bf16", 64), ("bf16", 128),
                                     ("bf16", 256), ("bf16", 512)])
def test_every_row_width(dtype, F):
    rng = np.random.default_rng(F)
    ip, ix = gg.random_multigraph(600, 4000, rng, hub_rows=(3, 77), hub_deg=700)
    x = gg.normal_features(rng, (600, F), dtype)
    dout = gg.normal_features(rng, (600, F), dtype)
    shuffled = ix.copy()                      # the same graph with rows in random order
    for i in range(600):
        rng.shuffle(shuffled[ip[i]:ip[i + 1]])
    for op in ("max", "min"):
        for tag, idx in (("sorted", ix), ("unsorted", shuffled)):
            plan, out, arg, ra = fwd_exact(f"width {F} {tag}", ip, idx, x, dtype, op,
                                           light_max_deg=4, hub_min_deg_exclusive=64,
                                           hub_chunk=40)
            assert plan.info()["rows_sorted"] == (tag == "sorted")
            bwd_parity(f"width {F} {op} {tag}", plan, ip, idx, arg, ra, dout, dtype)


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ties_signed_zeros_and_infinities(dtype, order):
    # values on a coarse grid (ties everywhere), with -0.0, +0.0, -inf and +inf mixed in,
    # on a multigraph with many parallel edges; neighbour lists sorted (the kernels' sorted
    # path) or in random order
    rng = np.random.default_rng(11)
    n, F = 300, 64
    ip, ix = gg.random_multigraph(n, 6000, rng, hub_rows=(7,), hub_deg=900)
    ix = ix.copy()
    if order == "shuffled":
        for i in range(n):
            rng.shuffle(ix[ip[i]:ip[i + 1]])
    xv = rng.integers(-2, 3, size=(n, F)).astype(np.float32)
    special = np.array([-0.0, 0.0, -np.inf, np.inf], np.float32)
    pick = rng.random((n, F)) < 0.15
    xv[pick] = special[rng.integers(0, 4, pick.sum())]
    x = gg.f32_to_bf16_bits(xv) if dtype == "bf16" else xv
    for op in ("max", "min"):
        for bins in ({}, dict(light_max_deg=2, hub_min_deg_exclusive=20, hub_chunk=7),
                     dict(light_max_deg=2, hub_min_deg_exclusive=20, hub_chunk=7,
                          xcd_split_min_deg_exclusive=10)):
            plan, out, arg, ra = fwd_exact(f"ties {dtype}", ip, ix, x, dtype, op, **bins)
            # backward: each parallel edge is one variable; gradient finite everywhere
            dout = gg.normal_features(rng, (n, F), dtype)
            bwd_parity(f"ties {dtype} {op}", plan, ip, ix, arg, ra, dout, dtype)


def test_empty_rows_and_graphs():
    rng = np.random.default_rng(5)
    ip, ix = gg.random_multigraph(500, 300, rng, self_loops=False)   # many empty rows
    assert (np.diff(ip) == 0).sum() > 100
    x = gg.normal_features(rng, (500, 128), "bf16")
    dout = gg.normal_features(rng, (500, 128), "bf16")
    for op in ("max", "min"):
        plan, out, arg, ra = fwd_exact("empty rows", ip, ix, x, "bf16", op)
        empty = torch.from_numpy(np.diff(ip) == 0).cuda()
        assert (arg[0][empty] == -1).all() and (out[empty] == 0).all()
        dx, _ = bwd_parity("empty rows", plan, ip, ix, arg, ra, dout, "bf16")
        nosrc = torch.from_numpy(np.bincount(ix, minlength=500) == 0).cuda()
        assert (dx[nosrc] == 0).all()
    # nodes but no edges: every row empty, every column empty
    say("no edges")
    plan = Plan(np.zeros(9, np.int32), np.zeros(0, np.int32)).upload()
    xt = torch.randn(8, 64, device="cuda")
    out, arg, slot = reduce_fwd(plan, xt, op="max")
    dx = reduce_bwd(plan, None, torch.randn(8, 64, device="cuda"), slot=slot)
    assert (out == 0).all() and (arg == -1).all() and (dx == 0).all() and (slot == -1).all()
    # no nodes at all
    say("no nodes")
    plan = Plan(np.zeros(1, np.int32), np.zeros(0, np.int32)).upload()
    z = torch.zeros((0, 64), device="cuda")
    out, arg, slot = reduce_fwd(plan, z)
    assert out.shape == (0, 64) and reduce_bwd(plan, arg, z, slot=slot).shape == (0, 64)


def test_deterministic_and_autograd():
    w = gg.WORKLOADS["chunglu1m_max_train_bf16"]
    ip, ix = gg.make_graph(w, n=20_000)
    (x,) = gg.make_features(w, n=20_000)
    say("determinism and autograd, chunglu20k bf16")
    plan = Plan(ip, ix, light_max_deg=8, hub_min_deg_exclusive=64, hub_chunk=32).upload()
    xt = dev(x).float().requires_grad_(True)
    g = torch.randn_like(xt)
    out, arg = graph_reduce(plan, xt, "max")
    out.backward(g)
    dx1 = reduce_bwd(plan, arg, g)
    assert torch.equal(xt.grad, dx1)
    out2, arg2, slot2 = reduce_fwd(plan, xt.detach(), op="max")
    dx2 = reduce_bwd(plan, None, g, slot=slot2)
    assert torch.equal(out, out2) and torch.equal(arg, arg2) and torch.equal(dx1, dx2)


@pytest.mark.slow
@pytest.mark.parametrize("plan_kw", [
    pytest.param({}, id="default-plan"),
    pytest.param(dict(xcd_split_min_deg_exclusive=512, col_xcd_split_min_deg_exclusive=512),
                 id="bench-split-plan")])
def test_full_chunglu1m_sampled(plan_kw):
    """Full workload size (the default plan and the bench's split plan): the forward on
    sampled rows (hub, medium and light), the backward on sampled columns (one of them a
    hub column), against the oracle computed row by row; and the gradient-mass identity
    over the whole graph."""
    w = gg.WORKLOADS["chunglu1m_max_train_bf16"]
    ip, ix = gg.make_graph(w)
    (x,) = gg.make_features(w)
    dout = gg.make_dout(w)
    N = ip.size - 1
    deg = np.diff(ip)
    rng = np.random.default_rng(0)
    hub_rows = np.argsort(-deg)[:3]
    med = rng.choice(np.nonzero((deg > 16) & (deg <= 1024))[0], 40, replace=False)
    light = rng.choice(np.nonzero(deg <= 16)[0], 40, replace=False)
    rows = np.concatenate([hub_rows, med, light])
    plan, out, (arg, slot), _ = fwd_exact("chunglu1m bf16 sampled", ip, ix, x, "bf16", "max",
                                          rows=rows, **plan_kw)
    assert slot.dtype == torch.int16
    say("chunglu1m backward sampled columns")
    dx = reduce_bwd(plan, None, dev(dout), slot=slot)
    torch.cuda.synchronize()
    colptr, rowidx = P.transpose(ip, ix)
    odeg = np.diff(colptr)
    hubc = np.nonzero((odeg > 1024) & (odeg < 3000))[0][:1]
    cols = np.concatenate([hubc, rng.choice(np.nonzero((odeg > 16) & (odeg <= 200))[0], 5,
                                            replace=False),
                           rng.choice(np.nonzero(odeg <= 16)[0], 10, replace=False)])
    ref, rrows, rarg = R.grad_cols_sampled(ip, ix, colptr, rowidx, x, dout, cols, "max")
    # the GPU's args of every row that feeds these columns equal the oracle's
    assert np.array_equal(arg[torch.from_numpy(rrows).cuda()].reshape(len(rrows), -1)
                          .cpu().numpy(), rarg)
    ct = torch.from_numpy(cols).cuda()
    check("chunglu1m dx sampled", host64(dx[ct]).reshape(ref.shape), ref, "bf16")
    # every (row, element) with a neighbour routes its gradient to exactly one source
    tot = host64(dx).reshape(N, -1).sum(0)
    dref = gg.bf16_bits_to_f32(dout).reshape(N, -1).astype(np.float64)[deg > 0].sum(0)
    scale = np.abs(host64(dx)).reshape(N, -1).sum(0)
    assert np.all(np.abs(tot - dref) <= 2 ** -8 * scale)


def test_wide_slots_for_rows_beyond_65535_edges():
    """A row with more than 65535 edges makes the slots 32-bit; forward and backward in
    both match modes, with parallel edges in the long row."""
    rng = np.random.default_rng(21)
    n = 4000
    src = np.concatenate([rng.integers(0, n, 70_000), rng.integers(0, n, 20_000)])
    dst = np.concatenate([np.full(70_000, 11), rng.integers(0, n, 20_000)])
    ip, ix = gg.csr_from_edges(n, src, dst)
    x = gg.normal_features(rng, (n, 32), "bf16")
    dout = gg.normal_features(rng, (n, 32), "bf16")
    for op in ("max", "min"):
        plan, out, arg_slot, ra = fwd_exact("wide slots", ip, ix, x, "bf16", op)
        assert reduce_slot_dtype(plan) == torch.int32 and arg_slot[1].dtype == torch.int32
        bwd_parity("wide slots", plan, ip, ix, arg_slot, ra, dout, "bf16")


def test_no_winner_slot_never_matches_a_position():
    """A row of exactly 65536 edges has positions up to 65535 = 0xFFFF, the 16-bit form of
    the all-ones slot of an element without a winner, so such a plan takes 32-bit slots.
    Here one feature column is NaN on every node: that element has no winner in any row,
    so its dx must stay exactly zero (with 16-bit slots the row's last edge would match);
    the other columns follow the oracle, run with that column set to zero."""
    rng = np.random.default_rng(23)
    n = 3000
    rs, rd = rng.integers(0, n, 9_000), rng.integers(0, n, 9_000)
    keep = (rd != 7) & (rs != rd)                # row 7 gets exactly the 65536 long-row edges
    src = np.concatenate([rng.integers(0, n, 65_536), rs[keep]])
    dst = np.concatenate([np.full(65_536, 7), rd[keep]])
    ip, ix = gg.csr_from_edges(n, src, dst)
    assert ip[8] - ip[7] == 65_536
    x = gg.f32_to_bf16_bits(rng.standard_normal((n, 32)).astype(np.float32))
    dout = gg.normal_features(rng, (n, 32), "bf16")
    c0 = 5
    xn = x.copy()
    xn[:, c0] = gg.f32_to_bf16_bits(np.full(n, np.nan, np.float32))
    x0 = x.copy()
    x0[:, c0] = 0
    say("no-winner slots, long row", ip[8] - ip[7], "E", ix.size)
    plan = Plan(ip, ix).upload()
    assert reduce_slot_dtype(plan) == torch.int32
    out, arg, slot = reduce_fwd(plan, dev(xn), op="max")
    dx = reduce_bwd(plan, None, dev(dout), slot=slot)
    torch.cuda.synchronize()
    assert torch.all(arg[:, c0] == -1) and torch.all(slot[:, c0] == -1)
    assert torch.all(dx[:, c0].float() == 0)
    _, ra = R.reduce_rows(ip, ix, x0, np.arange(n), "max")
    others = np.r_[0:c0, c0 + 1:32]
    assert np.array_equal(arg[:, others].cpu().numpy(), ra[:, others])
    rdx = R.reduce_backward(ra, dout, n)
    check("no-winner slots dx", host64(dx[:, others]), rdx[:, others], "bf16")


@pytest.mark.parametrize("dtype,F", [("bf16", 256), ("f32", 128), ("bf16", 64)])
def test_feature_slices(dtype, F):
    """Every slice count gives the same out, arg and slot bit for bit (selection is exact)
    and the oracle's dx."""
    rng = np.random.default_rng(41)
    ip, ix = gg.random_multigraph(800, 6000, rng, hub_rows=(5, 9), hub_deg=900)
    x = gg.normal_features(rng, (800, F), dtype)
    dout = gg.normal_features(rng, (800, F), dtype)
    first = None
    for S in (1, 2, 4, 8):
        plan, out, (arg, slot), ra = fwd_exact(f"slices {S} F{F}", ip, ix, x, dtype, "max",
                                               light_max_deg=4, hub_min_deg_exclusive=64,
                                               hub_chunk=40, feature_slices=S)
        bwd_parity(f"slices {S} F{F}", plan, ip, ix, (arg, slot), ra, dout, dtype)
        if first is None:
            first = (out, arg, slot)
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, (out, arg, slot)))


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
@pytest.mark.parametrize("op", ["max", "min"])
def test_rows_of_only_infinities_and_nan(op, order):
    """A row whose values are all -inf (max) or +inf (min) returns that infinity and the
    smallest id; NaN never wins, and a row of NaN only reads as empty."""
    inf = -np.inf if op == "max" else np.inf
    # node values: 0, 1, 3 = inf; 2 = NaN.  Rows: 0 <- {1, 2, 3} (inf, NaN, inf);
    # 1 <- {0, 2} (inf, NaN); 2 <- {2, 2} (NaN only, a parallel edge); 3 <- {} (empty)
    ip, ix = gg.csr_from_edges(4, np.array([1, 2, 3, 0, 2, 2, 2]),
                               np.array([0, 0, 0, 1, 1, 2, 2]))
    assert np.array_equal(ix, [1, 2, 3, 0, 2, 2, 2])
    if order == "shuffled":
        ix = np.array([3, 1, 2, 2, 0, 2, 2], dtype=ix.dtype)   # rows out of id order
    x = np.zeros((4, 16), np.float32)
    x[1] = x[3] = inf
    x[0] = inf
    x[2] = np.nan
    say("infinities and NaN", op, order)
    plan = Plan(ip, ix).upload()
    assert plan.info()["rows_sorted"] == (order == "sorted")
    out, arg, _ = reduce_fwd(plan, dev(x), op=op)
    o, a = out.cpu().numpy(), arg.cpu().numpy()
    assert np.all(o[0] == inf) and np.all(a[0] == 1)
    assert np.all(o[1] == inf) and np.all(a[1] == 0)
    assert np.all(o[2] == 0) and np.all(a[2] == -1)
    assert np.all(o[3] == 0) and np.all(a[3] == -1)


def test_full_split_plan_matches_the_bench():
    import bench
    assert bench.XCD_SPLIT_REDUCE == 512
