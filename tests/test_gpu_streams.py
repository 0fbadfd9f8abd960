"""One uploaded plan shared by calls on two streams at once: the plan is read-only after
upload, so concurrent calls with their own workspaces and outputs must give what the same
calls give one after the other, bit for bit (the kernels are deterministic)."""
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


@pytest.mark.parametrize("plan_kw", [
    pytest.param({}, id="default-plan"),
    pytest.param(dict(xcd_split_min_deg_exclusive=256, col_xcd_split_min_deg_exclusive=1024),
                 id="split-plan")])
def test_two_streams_share_a_plan(plan_kw):
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 30_000
    ip, ix = gg.make_graph(w, n=n)
    rng = np.random.default_rng(8)
    print("[case] two streams, one plan: N", n, "E", ix.size, flush=True)
    plan = ga.Plan(ip, ix, **plan_kw).upload()
    scale = 1 / math.sqrt(32)
    sets = [[dev(gg.normal_features(rng, (n, 8, 32), "bf16")) for _ in range(4)]
            for _ in range(2)]

    def step(q, k, v, do, stream):
        fws = torch.empty(max(plan.fwd_workspace_bytes(8, 32), 1), dtype=torch.uint8,
                          device="cuda")
        bws = torch.empty(plan.bwd_workspace_bytes(8, 32), dtype=torch.uint8, device="cuda")
        out, lse = ga.fwd(plan, q, k, v, scale=scale, workspace=fws, stream=stream)
        dq, dk, dv = ga.bwd(plan, q, k, v, do, lse, scale=scale, workspace=bws, stream=stream)
        return [out, lse, dq, dk, dv], (fws, bws)

    # one after the other on the default stream
    serial = [step(*s, None)[0] for s in sets]
    torch.cuda.synchronize()
    # at the same time on two side streams (buffers allocated up front on the current
    # stream, then both streams wait for that before they start)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results, keep = [], []
    for _ in range(3):                                  # several rounds of overlap
        for s, st in zip(sets, streams):
            with torch.cuda.stream(st):
                res, bufs = step(*s, st)
            results.append(res)
            keep.append(bufs)
    torch.cuda.synchronize()
    for r, res in enumerate(results):
        for a, b in zip(serial[r % 2], res):
            assert torch.equal(a, b), f"concurrent call {r} differs from the serial result"


def test_upload_again_retargets_the_plan():
    """A second upload moves the plan to a new device buffer. The first buffer is then
    zeroed (a zeroed plan reads as a graph whose rows and columns are all empty, so a
    plan still pointing there would give different results without reading out of
    bounds): fwd and bwd must give what they gave before, bit for bit."""
    w = gg.WORKLOADS["chunglu1m_train_bf16"]
    n = 5_000
    ip, ix = gg.make_graph(w, n=n)
    rng = np.random.default_rng(12)
    print("[case] plan uploaded twice: N", n, "E", ix.size, flush=True)
    q, k, v, do = (dev(gg.normal_features(rng, (n, 8, 32), "bf16")) for _ in range(4))
    plan = ga.Plan(ip, ix, hub_min_deg_exclusive=64, hub_chunk=32).upload()
    out1, lse1 = ga.fwd(plan, q, k, v)
    g1 = ga.bwd(plan, q, k, v, do, lse1)
    torch.cuda.synchronize()
    first = plan.device_buffer
    plan.upload()
    assert plan.device_buffer.data_ptr() != first.data_ptr()
    first.zero_()
    out2, lse2 = ga.fwd(plan, q, k, v)
    g2 = ga.bwd(plan, q, k, v, do, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
