"""The largest graph the library takes: E = 2^31 - 2^16 edges (the planner rejects one more),
so the last rows' and the hub chunks' edge positions come within 2^16 of the 32-bit signed
range the kernels walk them in, and the transpose's column positions span the same range.

1M nodes: 10% light rows (0..16 edges), eight 4M-edge hub rows (four at the very end of the
edge range), the rest medium rows of ~2,300 edges. Each row's sources are a stratified
sample of the node range, so every neighbour list is sorted (hub rows repeat each source
about four times: runs of parallel edges). bf16 features, H = 2, d = 32. The dot training
step runs on the default plan; the oracle checks out, lse and dq on sampled rows (the first
and last rows, two hubs, random rows) and dk, dv on sampled columns (every edge into them,
hub rows included). The max-pooling forward runs on the same plan (sorted rows: the
kernels' reversed edge order) and its out, arg and slot must match exactly on the rows.
"""
import math

import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A
from oracle import reduction as R
from sparse_graph_attention_02_amd import Plan, bwd, fwd, reduce_fwd
from tests.gpu_util import check, check_lse, dev, host64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

KMAX = (1 << 31) - (1 << 16)
N = 1 << 20
H, D = 2, 32
HUB = 1 << 22


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def say(*a):
    print("[case]", *a, flush=True)


def max_graph(n=N, e=KMAX, hub=HUB, seed=31):
    """CSR of n nodes and exactly e edges: 10% light rows, eight hub rows of `hub` edges
    (rows n/2, n-64, n-2, n-1 and four random ones), medium rows filling the rest. Row i's
    k-th source is floor((k + u) n / deg_i), u uniform in [0, 1): sorted within the row."""
    rng = np.random.default_rng(seed)
    deg = rng.integers(1200, 2800, n).astype(np.int64)
    light = rng.choice(n, n // 10, replace=False)
    deg[light] = rng.integers(0, 17, light.size)
    hubs = np.unique(np.concatenate([[n // 2, n - 64, n - 2, n - 1],
                                     rng.choice(n, 4, replace=False)]))
    deg[hubs] = hub
    med = np.setdiff1d(np.arange(n), np.concatenate([light, hubs]))
    q, rem = divmod(int(e - deg.sum()), med.size)
    deg[med] += q
    deg[med[:rem]] += 1
    assert deg.sum() == e and deg.min() >= 0 and deg[med].max() < 8192
    ip = np.zeros(n + 1, np.int64)
    np.cumsum(deg, out=ip[1:])
    ix = np.empty(e, np.int32)
    step = 1 << 15
    for r0 in range(0, n, step):                 # in row blocks, to bound the temporaries
        r1 = min(n, r0 + step)
        d = deg[r0:r1]
        a, b = int(ip[r0]), int(ip[r1])
        k = np.arange(b - a, dtype=np.int64) - np.repeat(ip[r0:r1] - a, d)
        dd = np.repeat(d, d).astype(np.float64)
        src = ((k + rng.random(b - a)) * (n / dd)).astype(np.int64)
        ix[a:b] = np.minimum(src, n - 1)
    return ip.astype(np.int32), ix, hubs


@pytest.mark.timeout(1200)
def test_dot_training_step_at_the_edge_limit():
    ip, ix, hubs = max_graph()
    say(f"N {N} E {int(ip[-1])} (limit {KMAX}) hubs {hubs.tolist()}")
    assert int(ip[-1]) == KMAX
    rng = np.random.default_rng(5)
    q, k, v, dout = (gg.f32_to_bf16_bits(rng.standard_normal((N, H, D), dtype=np.float32))
                     for _ in range(4))
    scale = float(np.float32(1 / math.sqrt(D)))
    plan = Plan(ip, ix).upload()
    info = plan.info()
    assert info["rows_sorted"]
    say("plan", {k_: info[k_] for k_ in ("n_row_light", "n_row_medium", "n_row_hub",
                                        "n_row_chunks", "max_in_degree")})
    assert info["n_row_hub"] == hubs.size
    tq, tk, tv, td = dev(q), dev(k), dev(v), dev(dout)
    out, lse = fwd(plan, tq, tk, tv, scale=scale)
    dq, dk, dv = bwd(plan, tq, tk, tv, td, lse, scale=scale)
    x = gg.f32_to_bf16_bits(np.round(rng.standard_normal((N, 32), dtype=np.float32) * 4) / 4)
    pout, parg, pslot = reduce_fwd(plan, dev(x), op="max")
    torch.cuda.synchronize()
    del tq, tk, tv, td, plan
    torch.cuda.empty_cache()

    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 3, N - 1],
                                     rng.choice(N, 40, replace=False)]))
    ro, rl, rq, _, _, _ = A.train_step_rows(ip, ix, q, k, v, dout, rows, scale)
    rt = torch.from_numpy(rows).cuda()
    for name, g, r in (("out", out, ro), ("dq", dq, rq)):
        say(name, check(name, host64(g[rt]), r, "bf16"))
    check_lse("lse", host64(lse[rt]), rl)

    # max pooling on the same rows: values on a coarse grid, so ties (and the parallel
    # edges of the hubs) exercise the smallest-id rule
    po, pa = R.reduce_rows(ip, ix, x, rows, "max")
    ps = R.slots_of(ip, ix, rows, pa)
    go = pout[rt].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(go, gg.f32_to_bf16_bits(po.astype(np.float32))), "pool out"
    assert np.array_equal(parg[rt].cpu().numpy().astype(np.int64), pa), "pool arg"
    gs = pslot[rt].cpu().numpy()
    gs = gs.view(np.uint16).astype(np.int64) if gs.dtype == np.int16 else gs.astype(np.int64)
    gs[gs == (0xFFFF if pslot.dtype == torch.int16 else -1)] = -1
    assert np.array_equal(gs, ps), "pool slot"
    say("pool out, arg, slot exact on", rows.size, "rows")

    cols = np.sort(rng.choice(N, 4, replace=False))
    rk, rv = A.grad_kv_cols(ip, ix, q, k, v, dout, cols, scale)
    ct = torch.from_numpy(cols).cuda()
    for name, g, r in (("dk", dk, rk), ("dv", dv, rv)):
        say(name, check(name, host64(g[ct]), r, "bf16"))
