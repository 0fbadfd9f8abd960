"""Host-side parts of bench.py: the one-GPU guard, the algorithmic byte model behind
`roofline.achieved`, and the node-order relabelling of the ablation."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import graphgen as gg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# Per edge and per node, written out by hand for each kernel (F = H d, b bytes per
# element): 4 bytes of index per edge and 4 of indptr per node, then one read of every
# gathered row per edge, every per-node operand once and every output once.
def _hand(kernel, H, d, b):
    F = H * d
    row = F * b
    table = {
        # kernel: (bytes per edge, bytes per node, constant)
        "fwd_main": (4 + 2 * row, 4 + row + row + 4 * H, 4),                    # K,V | Q,out,lse
        "bwd_dq_main": (4 + 2 * row, 4 + 2 * row + 4 * H + row + 8 * H, 4),     # K,V | Q,dO,lse,dQ,rec
        "bwd_dkdv_main": (4 + 2 * row + 8 * H, 4 + 2 * row + 2 * row, 4),       # Q,dO,rec | K,V,dK,dV
        "bwd_gat_rows_main": (4 + 4 * H + row, 4 + 4 * H + row + 4 * H + 4 * H + 8 * H, 4),
        # t_j, V_j | s, dO, lse, ds, record
        "bwd_gat_cols_main": (4 + 4 * H + row + 8 * H, 4 + 4 * H + row + 4 * H + row, 4),
        # s_i, dO_i, record_i | t, V, dt, dV
        "bwd_gatv2_rows_main": (4 + row, 4 + 2 * row + 4 * H + row + 8 * H, 4 + 4 * F),
        "bwd_gatv2_cols_main": (4 + 2 * row + 8 * H, 4 + row + row, 4 + 4 * F),
        "reduce_fwd_main": (4 + row, 4 + row + 4 * F + 2 * F, 4),             # x | out,arg,slot
        "reduce_bwd_main": (4 + 4 + 2 * F, 4 + row + row, 4),                  # rowidx,rel,slots | dO,dx
    }
    return table[kernel]


@pytest.mark.parametrize("kernel", ["fwd_main", "bwd_dq_main", "bwd_dkdv_main",
                                    "bwd_gat_rows_main", "bwd_gat_cols_main",
                                    "bwd_gatv2_rows_main", "bwd_gatv2_cols_main",
                                    "reduce_fwd_main", "reduce_bwd_main"])
@pytest.mark.parametrize("N,E,H,d,b", [(1_000_000, 50_997_829, 8, 32, 2),
                                       (2_097_152, 65_008_926, 1, 128, 2), (10, 0, 4, 16, 4)])
def test_byte_model_per_edge_and_node(kernel, N, E, H, d, b):
    score = ("gatv2" if "gatv2" in kernel else "gat" if "_gat_" in kernel
             else "max" if kernel.startswith("reduce") else "dot")
    pe, pn, c = _hand(kernel, H, d, b)
    assert bench.algorithmic_bytes(kernel, N, E, H, d, b, score) == pe * E + pn * N + c


def test_byte_model_figures_of_the_configurations():
    """Per-edge / per-node byte figures worked out by hand from the layouts: 1,028 / 1,060 B
    for the 1M forward; 1,044 / 1,060 B for the GAT forward (fp32, H = 4, d = 64); 516 / 520 B for
    the R-MAT forward; the 1M dK/dV pass 1,092 B per edge."""
    f = bench.algorithmic_bytes
    assert f("fwd_main", 1, 1, 8, 32, 2) - f("fwd_main", 1, 0, 8, 32, 2) == 1028
    assert f("fwd_main", 1, 0, 8, 32, 2) - f("fwd_main", 0, 0, 8, 32, 2) == 1060
    assert f("fwd_main", 1, 1, 4, 64, 4, "gat") - f("fwd_main", 1, 0, 4, 64, 4, "gat") == 1044
    assert f("fwd_main", 1, 0, 4, 64, 4, "gat") - f("fwd_main", 0, 0, 4, 64, 4, "gat") == 1060
    assert f("fwd_main", 1, 1, 1, 128, 2) - f("fwd_main", 1, 0, 1, 128, 2) == 516
    assert f("fwd_main", 1, 0, 1, 128, 2) - f("fwd_main", 0, 0, 1, 128, 2) == 520
    assert f("bwd_dkdv_main", 1, 1, 8, 32, 2) - f("bwd_dkdv_main", 1, 0, 8, 32, 2) == 1092
    # the whole training step is the sum of its three passes
    N, E = 1000, 5000
    assert bench.step_bytes(N, E, 8, 32, 2, True) == sum(
        f(k, N, E, 8, 32, 2) for k in ("fwd_main", "bwd_dq_main", "bwd_dkdv_main"))
    assert bench.step_bytes(N, E, 4, 64, 4, True, "gat") == sum(
        f(k, N, E, 4, 64, 4, "gat") for k in ("fwd_main", "bwd_gat_rows_main",
                                              "bwd_gat_cols_main"))


@pytest.mark.parametrize("order", ["random", "out-degree", "rcm"])
def test_relabel_keeps_the_graph_and_moves_node_arrays(order):
    rng = np.random.default_rng(4)
    n = 300
    ip, ix = gg.random_multigraph(n, 2500, rng, hub_rows=(7,), hub_deg=200)
    x = rng.standard_normal((n, 2, 4)).astype(np.float32)
    attn = rng.standard_normal((2, 4)).astype(np.float32)     # per graph: must stay
    dout = rng.standard_normal((n, 2, 4)).astype(np.float32)
    perm = {"random": lambda: rng.permutation(n),
            "out-degree": lambda: bench.order_by_out_degree(ip, ix),
            "rcm": lambda: bench.order_rcm(ip, ix)}[order]()
    assert np.array_equal(np.sort(perm), np.arange(n))
    ip2, ix2, (x2, a2), d2 = bench.relabel(ip, ix, (x, attn), dout, perm)
    assert np.array_equal(x2, x[perm]) and np.array_equal(d2, dout[perm])
    assert a2 is attn
    new_of_old = np.empty(n, np.int64)
    new_of_old[perm] = np.arange(n)
    dst = np.repeat(np.arange(n), np.diff(ip))
    before = sorted(zip(new_of_old[dst].tolist(), new_of_old[ix].tolist()))
    dst2 = np.repeat(np.arange(n), np.diff(ip2))
    assert before == sorted(zip(dst2.tolist(), ix2.tolist()))
    if order == "out-degree":
        odeg = np.bincount(ix2, minlength=n)
        assert np.all(np.diff(odeg) <= 0)


def test_xcd_split_defaults_of_the_workloads():
    W = gg.WORKLOADS
    assert bench.xcd_split_of(W["chunglu1m_train_bf16"]) == (256, 1024)
    assert bench.xcd_split_of(W["rmat21_dot_bf16"]) == (256, 1024)
    assert bench.xcd_split_of(W["chunglu1m_gatv2_train_bf16"]) == (256, 1024)
    assert bench.xcd_split_of(W["chunglu1m_max_train_bf16"]) == (512, 512)
    assert bench.xcd_split_of(W["chunglu1m_train_bf16"], 0) == (0, 0)
    assert bench.xcd_split_of(W["chunglu1m_train_bf16"], 2048) == (2048, 2048)
    assert bench.xcd_split_of(W["chunglu1m_train_bf16"], 128, 0) == (128, 0)
