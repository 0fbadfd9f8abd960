"""The gathers' 64-bit path (plain loads, taken for node tables past 4 GiB) on every compiled
geometry, at small sizes: GRAPH_ATTN_WIDE_LOADS=1 makes every call take it, and the
existing every-element parity cases run again under it. The forward (dot, GAT-style,
GATv2, with feature slices and on split plans), the GATv2 backward and the min / max
forward are the calls whose gathers have the two paths. A last case runs a whole set of
calls on both paths and requires equal outputs, element for element.
"""
import pytest
import torch

from tests import test_gpu_parity as P
from tests import test_gpu_reduce as R
from tests import test_gpu_xcd_split as X

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


@pytest.fixture(autouse=True)
def wide(monkeypatch):
    monkeypatch.setenv("GRAPH_ATTN_WIDE_LOADS", "1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", P.GEOMS)
def test_forward_geometries_wide(dtype, G, LH):
    P.test_every_compiled_geometry(dtype, G, LH)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", P.GEOMS)
def test_gatv2_forward_geometries_wide(dtype, G, LH):
    P.test_gatv2_forward_geometries(dtype, G, LH)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", P.GEOMS)
def test_gatv2_backward_geometries_wide(dtype, G, LH):
    P.test_gatv2_backward_every_element(dtype, G, LH)


@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype,H,d", [("bf16", 8, 32), ("f32", 4, 32), ("bf16", 2, 128)])
def test_forward_feature_slices_wide(S, dtype, H, d):
    P.test_feature_slices_every_element(S, dtype, H, d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_plans_wide(dtype):
    X.test_split_gat_and_gatv2_every_element(dtype)
    X.test_split_dot_forward_backward_every_element(dtype, 8)


@pytest.mark.parametrize("dtype,F", [("f32", 16), ("f32", 256), ("bf16", 32), ("bf16", 512)])
def test_reduction_widths_wide(dtype, F):
    R.test_every_row_width(dtype, F)


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reduction_ties_wide(dtype, order):
    R.test_ties_signed_zeros_and_infinities(dtype, order)


@pytest.fixture
def both_paths(monkeypatch):
    """Run fn twice, on the buffer-load path and on the 64-bit one; return both results."""
    def run(fn):
        monkeypatch.delenv("GRAPH_ATTN_WIDE_LOADS", raising=False)
        a = fn()
        monkeypatch.setenv("GRAPH_ATTN_WIDE_LOADS", "1")
        b = fn()
        torch.cuda.synchronize()
        return a, b
    return run


@pytest.mark.parametrize("plan_kw", [dict(light_max_deg=6, hub_min_deg_exclusive=40, hub_chunk=24),
                                     dict(xcd_split_min_deg_exclusive=16,
                                          col_xcd_split_min_deg_exclusive=16)],
                         ids=["bins", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_both_gather_paths_agree_exactly(dtype, plan_kw, both_paths):
    """The two gather paths run the same arithmetic in the same order, and a step's unused
    slots add exact zeros on both (a zero row, or a neighbour's row with weight zero), so
    every output is equal element for element (compared as values: a sum that is exactly
    zero may carry either sign)."""
    import numpy as np
    import graphgen as gg
    from sparse_graph_attention_02_amd import (Plan, bwd, bwd_gatv2, fwd, fwd_gatv2,
                                               reduce_fwd)
    from tests.gpu_util import dev
    rng = np.random.default_rng(3)
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n, H, d = 8000, 4, 32
    ip, ix = gg.make_graph(w, n=n)
    x = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(4)]
    if dtype == "bf16":
        x = [gg.f32_to_bf16_bits(y) for y in x]
    q, k, v, do = (dev(y) for y in x)
    s, t = (torch.from_numpy(rng.standard_normal((n, H)).astype(np.float32)).cuda()
            for _ in range(2))
    a = torch.from_numpy((rng.standard_normal((H, d)) / 8).astype(np.float32)).cuda()
    plan = Plan(ip, ix, **plan_kw).upload()
    P.say("gather paths agree", dtype, plan_kw)

    def step():
        out, lse = fwd(plan, q, k, v)
        g = bwd(plan, q, k, v, do, lse)
        gout, glse = fwd(plan, s, t, v, score="gat", scale=1.0)
        vout, vlse = fwd_gatv2(plan, q, k, a)
        vg = bwd_gatv2(plan, q, k, a, do, vlse)
        r = reduce_fwd(plan, v.reshape(n, H * d), op="max")
        return (out, lse, *g, gout, glse, vout, vlse, *vg, *r)

    first, second = both_paths(step)
    for i, (u, w_) in enumerate(zip(first, second)):
        assert torch.equal(u, w_), f"output {i} differs between the gather paths"
