"""Every row length from 0 to 200 edges, every element against the oracle.

The passes fold a row's edges in steps of U edges per lane group and fetch its neighbour
indices in batches of one per lane; the GATv2 row pass cuts its batches to whole steps,
runs full steps unmasked and skips the unused slots of an item's last step, and in the
narrowest geometries a step is wider than a batch. A "staircase" graph whose rows hold
0, 1, ..., 200 edges (then a second ramp) meets every residue of every step and batch
length in light rows, medium rows and hub chunks (chunks of 37 edges, a length no step
divides). Each case runs on the buffer-load path and on the 64-bit one.
"""
import numpy as np
import pytest
import torch

import graphgen as gg
from tests import test_gpu_parity as P

pytestmark = pytest.mark.gpu

GEOMS = [(4, 2), (4, 4), (8, 4), (16, 4), (32, 4), (32, 8), (64, 16)]
PLANS = {"default": {}, "hub-chunks": dict(light_max_deg=16, hub_min_deg_exclusive=64,
                                           hub_chunk=37)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


@pytest.fixture(params=["buffer", "wide"])
def path(request, monkeypatch):
    if request.param == "wide":
        monkeypatch.setenv("GRAPH_ATTN_WIDE_LOADS", "1")
    return request.param


def staircase(seed):
    """CSR over 320 nodes: row i holds i edges for i <= 200, then rows of 0..119 edges;
    sources uniform over all nodes (parallel edges allowed)."""
    rng = np.random.default_rng(seed)
    n = 320
    deg = np.r_[np.arange(201), np.arange(n - 201)]
    rng.shuffle(deg[201:])
    ip = np.zeros(n + 1, np.int64)
    np.cumsum(deg, out=ip[1:])
    ix = rng.integers(0, n, int(ip[-1])).astype(np.int32)
    return ip.astype(np.int32), ix


def feats(rng, n, H, d, dtype, k):
    x = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(k)]
    return [gg.f32_to_bf16_bits(y) for y in x] if dtype == "bf16" else x


def shape_of(G, LH, dtype):
    eb = 4 if dtype == "f32" else 2
    return G // LH, LH * 16 // eb


@pytest.mark.parametrize("plan_name", list(PLANS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_dot_every_row_length(G, LH, dtype, plan_name, path):
    H, d = shape_of(G, LH, dtype)
    ip, ix = staircase(G * 7 + LH)
    rng = np.random.default_rng(G + LH)
    q, k, v, do = feats(rng, ip.size - 1, H, d, dtype, 4)
    P.fwd_parity(f"staircase dot G{G} LH{LH} {dtype} {plan_name} {path}", ip, ix, q, k, v,
                 dtype, **PLANS[plan_name])
    P.bwd_case(f"staircase dot bwd G{G} LH{LH} {dtype} {plan_name} {path}", ip, ix, q, k, v,
               do, dtype, **PLANS[plan_name])


@pytest.mark.parametrize("plan_name", list(PLANS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", GEOMS)
def test_gatv2_every_row_length(G, LH, dtype, plan_name, path):
    H, d = shape_of(G, LH, dtype)
    ip, ix = staircase(G * 11 + LH)
    rng = np.random.default_rng(G * 3 + LH)
    xd, xs, do = feats(rng, ip.size - 1, H, d, dtype, 3)
    a = (rng.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    tag = f"staircase gatv2 G{G} LH{LH} {dtype} {plan_name} {path}"
    P.gatv2_fwd_case(tag, ip, ix, xd, xs, a, dtype, scale=1.1, slope=0.2, **PLANS[plan_name])
    P.gatv2_bwd_case(tag + " bwd", ip, ix, xd, xs, a, do, dtype, scale=1.1, slope=0.2,
                     **PLANS[plan_name])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,LH", [(8, 8), (32, 32), (64, 64)])
def test_gat_every_row_length(G, LH, dtype, path):
    H, d = shape_of(G, LH, dtype)
    ip, ix = staircase(G * 5 + 1)
    rng = np.random.default_rng(G * 9)
    n = ip.size - 1
    s, t = (rng.standard_normal((n, H)).astype(np.float32) for _ in range(2))
    v, do = feats(rng, n, H, d, dtype, 2)
    for plan_name, kw in PLANS.items():
        tag = f"staircase gat G{G} LH{LH} {dtype} {plan_name} {path}"
        P.fwd_parity(tag, ip, ix, s, t, v, dtype, score="gat", scale=1.0, **kw)
        P.gat_bwd_case(tag + " bwd", ip, ix, s, t, v, do, dtype, **kw)
