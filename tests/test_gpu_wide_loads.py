"""The gathers' 64-bit path (plain loads, taken for node tables past 4 GiB) on every compiled
geometry, at small sizes: GRAPH_ATTN_WIDE_LOADS=1 makes every call take it, and the
existing every-element parity cases run again under it. The forward (dot, GAT-style,
GATv2, with feature slices and on split plans), the GATv2 backward and the min / max
forward are the calls whose gathers have the two paths.
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
