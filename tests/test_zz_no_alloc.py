"""GPU: the allocation-free forward (graph_attn_fwd_noalloc, through the C ABI) against the
forward with a caller workspace (graph_attn_fwd) and the fp64 oracle, on two calls in a
row, the second with a smaller input, so the second runs on the scratch the first left.

The two entry points run the same kernels, so their results must agree bit for bit; both
are also held to the parity criteria against the oracle.
"""
import math

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A
from sparse_graph_attention_02_amd import Plan, capi, fwd, fwd_noalloc
from tests.gpu_util import check, check_lse, dev, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def say(*a):
    print("[case]", *a, flush=True)


def _one(tag, ip, ix, a, b, v, dtype, score, scale, **plan_kw):
    H, d = v.shape[1], v.shape[2]
    say(tag, "N", ip.size - 1, "E", ix.size, "H", H, "d", d, dtype, score, plan_kw)
    plan = Plan(ip, ix, build_csc=False, **plan_kw).upload()
    need = plan.fwd_workspace_bytes(H, d)
    assert 0 < need <= capi.GA_FWD_NOALLOC_SCRATCH_BYTES
    ta, tb, tv = dev(a), dev(b), dev(v)
    out = torch.empty_like(tv)
    lse = torch.empty((ip.size - 1, H), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fwd_noalloc(plan, ta, tb, tv, score=score, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before      # nothing allocated by the call
    ref_out, ref_lse = fwd(plan, ta, tb, tv, score=score, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       ref_out.view(torch.int16) if out.dtype == torch.bfloat16
                       else ref_out.view(torch.int32)), f"{tag}: out differs from graph_attn_fwd"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), \
        f"{tag}: lse differs from graph_attn_fwd"
    ro, rl = A.forward(ip, ix, a, b, v, score, scale)
    check(f"{tag} out", host64(out), ro, dtype)
    check_lse(f"{tag} lse", host64(lse), rl)
    return need


def test_noalloc_forward_two_calls_second_smaller():
    w = gg.WORKLOADS["chunglu1m_dot_bf16"]
    n1 = 20_000
    ip, ix = gg.make_graph(w, n=n1)
    q, k, v = gg.make_features(w, n=n1)
    scale = float(np.float32(1 / math.sqrt(w.dim)))
    need1 = _one("noalloc call 1: chunglu20k bf16 dot", ip, ix, q, k, v, "bf16", "dot", scale,
                 light_max_deg=8, hub_min_deg_exclusive=64, hub_chunk=64,
                 xcd_split_min_deg_exclusive=64)     # 23 MB of hub partials
    # second call: a smaller graph, another dtype and score, on the scratch call 1 left
    rng = np.random.default_rng(11)
    n2 = 3000
    ip2, ix2 = gg.random_multigraph(n2, 40_000, rng, hub_rows=(7, 100), hub_deg=4000)
    s = rng.standard_normal((n2, 4)).astype(np.float32)
    t = rng.standard_normal((n2, 4)).astype(np.float32)
    v2 = rng.standard_normal((n2, 4, 16)).astype(np.float32)
    need2 = _one("noalloc call 2: random 3k f32 gat", ip2, ix2, s, t, v2, "f32", "gat", 1.0,
                 light_max_deg=4, hub_min_deg_exclusive=32, hub_chunk=8)
    assert need2 < need1
