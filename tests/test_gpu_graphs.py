"""HIP-graph capture of whole training steps: the library allocates nothing and records no
memset, so a step captures into a graph. Each graph is replayed several times, with
unrelated eager work and synchronisations between replays, and every replay must equal the
eager result bit for bit (the kernels are deterministic)."""
import math

import numpy as np
import pytest
import torch

import graphgen as gg
import sparse_graph_attention_02_amd as ga
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def say(*a):
    print("[case]", *a, flush=True)


def _replays_match(step, outputs, noise, reps=3):
    """Eager reference, capture, then replays separated by eager work."""
    ga.timers(enable=False, reset=True)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                    # warm-up on a side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(reps):
        for t in outputs:
            t.fill_(-7)                           # eager kernels between replays
        noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outputs)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager step"


def _graph(n=20_000):
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    return gg.make_graph(w, n=n)


# plans: the library default, and the XCD split bench.py uses for the attention workloads
PLANS = [pytest.param({}, id="default-plan"),
         pytest.param(dict(xcd_split_min_deg_exclusive=256,
                           col_xcd_split_min_deg_exclusive=1024), id="split-plan")]


@pytest.mark.parametrize("plan_kw", PLANS)
def test_dot_training_step_captures(plan_kw):
    ip, ix = _graph()
    n = ip.size - 1
    rng = np.random.default_rng(1)
    q, k, v, do = (dev(gg.normal_features(rng, (n, 8, 32), "bf16")) for _ in range(4))
    say("graph capture: dot training step, N", n, "E", ix.size, plan_kw)
    plan = ga.Plan(ip, ix, **plan_kw).upload()
    out, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((n, 8), device="cuda")
    fws = torch.empty(max(plan.fwd_workspace_bytes(8, 32), 1), dtype=torch.uint8, device="cuda")
    bws = torch.empty(plan.bwd_workspace_bytes(8, 32), dtype=torch.uint8, device="cuda")
    scale = 1 / math.sqrt(32)

    def step():
        ga.fwd(plan, q, k, v, scale=scale, out=out, lse=lse, workspace=fws)
        ga.bwd(plan, q, k, v, do, lse, scale=scale, dq=dq, dk=dk, dv=dv, workspace=bws)

    x = torch.randn(4096, 4096, device="cuda")
    _replays_match(step, [out, lse, dq, dk, dv], lambda: (x @ x).sum().item())


@pytest.mark.parametrize("plan_kw", PLANS)
def test_gatv2_training_step_captures(plan_kw):
    ip, ix = _graph()
    n = ip.size - 1
    rng = np.random.default_rng(2)
    xd, xs, do = (dev(gg.normal_features(rng, (n, 8, 32), "bf16")) for _ in range(3))
    attn = torch.from_numpy(rng.standard_normal((8, 32)).astype(np.float32) / 6).cuda()
    say("graph capture: GATv2 training step, N", n, "E", ix.size, plan_kw)
    plan = ga.Plan(ip, ix, **plan_kw).upload()
    out, dxd, dxs = (torch.empty_like(xs) for _ in range(3))
    lse = torch.empty((n, 8), device="cuda")
    dattn = torch.empty((8, 32), device="cuda")
    fws = torch.empty(max(plan.fwd_workspace_bytes(8, 32), 1), dtype=torch.uint8, device="cuda")
    bws = torch.empty(ga.bwd_gatv2_workspace_bytes(plan, xs.dtype, 8, 32), dtype=torch.uint8,
                      device="cuda")

    def step():
        ga.fwd_gatv2(plan, xd, xs, attn, out=out, lse=lse, workspace=fws)
        ga.bwd_gatv2(plan, xd, xs, attn, do, lse, dxd=dxd, dxs=dxs, dattn=dattn, workspace=bws)

    _replays_match(step, [out, lse, dxd, dxs, dattn], lambda: torch.cuda.synchronize())


@pytest.mark.parametrize("plan_kw", [
    pytest.param({}, id="default-plan"),
    pytest.param(dict(xcd_split_min_deg_exclusive=512, col_xcd_split_min_deg_exclusive=512),
                 id="split-plan")])
def test_reduction_training_step_captures(plan_kw):
    ip, ix = _graph()
    n = ip.size - 1
    rng = np.random.default_rng(3)
    x, do = (dev(gg.normal_features(rng, (n, 256), "bf16")) for _ in range(2))
    say("graph capture: max-pooling training step, N", n, "E", ix.size, plan_kw)
    plan = ga.Plan(ip, ix, **plan_kw).upload()
    out = torch.empty_like(x)
    arg = torch.empty(x.shape, dtype=torch.int32, device="cuda")
    slot = torch.empty(x.shape, dtype=ga.reduce_slot_dtype(plan), device="cuda")
    dx = torch.empty_like(x)
    from ctypes import byref, c_size_t
    b = c_size_t()
    ga.capi.graph_attn_reduce_fwd_workspace_bytes(plan.handle, 256, byref(b))
    fws = torch.empty(max(b.value, 1), dtype=torch.uint8, device="cuda")
    ga.capi.graph_attn_reduce_bwd_workspace_bytes(plan.handle, 256, byref(b))
    bws = torch.empty(max(b.value, 1), dtype=torch.uint8, device="cuda")

    def step():
        ga.reduce_fwd(plan, x, op="max", out=out, arg=arg, slot=slot, workspace=fws)
        ga.reduce_bwd(plan, None, do, slot=slot, dx=dx, workspace=bws)

    _replays_match(step, [out, arg, slot, dx], lambda: ga.reduce_fwd(plan, x, op="min"))
