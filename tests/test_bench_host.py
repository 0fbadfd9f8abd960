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
    # the plan options: dot-score split transposes take 1024-edge column chunks
    assert bench.bench_plan_kw(W["chunglu1m_train_bf16"]) == dict(
        xcd_split_min_deg_exclusive=256, col_xcd_split_min_deg_exclusive=1024, col_hub_chunk=1024)
    assert bench.bench_plan_kw(W["chunglu1m_gatv2_train_bf16"]) == dict(
        xcd_split_min_deg_exclusive=256, col_xcd_split_min_deg_exclusive=1024)
    assert bench.bench_plan_kw(W["chunglu1m_train_bf16"], 0) == dict(
        xcd_split_min_deg_exclusive=0, col_xcd_split_min_deg_exclusive=0)
    assert bench.bench_plan_kw(W["chunglu1m_train_bf16"], col_chunk=512)["col_hub_chunk"] == 512


def _fake_run(tmp, workload="chunglu1m_train_bf16", fetch_copy=524288, write_copy=1048576,
              fetch_k=1_000_000, write_k=20_000):
    """A directory shaped like the rocprofv3 runs of bench.py: the kernel-trace run's log
    and stats, and two counter passes (FETCH_SIZE, WRITE_SIZE) with the copy kernel."""
    import json
    run = tmp / "run"
    plan = {k: i for i, k in enumerate(bench.PLAN_KEYS)}
    line = {"ms_per_step": 10.0, "value": 1e9, "dtype": "bf16",
            "config": {"workload": workload, "nodes": 1000, "edges": 5000, "heads": 8,
                       "dim": 32, "score": "dot", "step": "forward+backward",
                       "node_order": "as-generated", "plan": plan},
            "kernels": {"fwd_main": {"avg_ms": 0.5}}}
    (run / "kt" / "host").mkdir(parents=True)
    (run / "kt.log").write_text("[bench] noise\n" + json.dumps(line) + "\n")
    name_k = "void ga::(anonymous namespace)::fwd_main<unsigned short, 32, 4, 0, 8>(ga::FwdArgs)"
    (run / "kt" / "host" / "kt_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        f'"{name_k}",10,5000000,500000,90.0,490000,510000,1.0\n'
        '"void ga::(anonymous namespace)::copy_probe(HIP_vector_type<unsigned int, 4u>*)",'
        '3,1200000,400000,10.0,390000,410000,1.0\n')
    for k, (ctr, vcopy, vk) in enumerate((("FETCH_SIZE", fetch_copy, fetch_k),
                                          ("WRITE_SIZE", write_copy, write_k)), 1):
        d = run / f"p{k}" / "host"
        d.mkdir(parents=True)
        rows = ['"Kernel_Name","Counter_Name","Counter_Value"']
        rows += [f'"{name_k}","{ctr}",{vk}', f'"{name_k}","{ctr}",{vk}',
                 f'"copy_probe","{ctr}",{vcopy}']
        (d / f"p{k}_counter_collection.csv").write_text("\n".join(rows) + "\n")
        (run / f"p{k}.counters").write_text(ctr + "\n")
    return run, plan


def test_counter_ingest_calibrates_on_the_copy_kernel(tmp_path):
    """FETCH_SIZE counts 64 bytes per 128-byte request on this part: the copy kernel moving
    1 GiB each way reads 524,288 KiB fetched and 1,048,576 KiB written, so the factors are
    2 and 1, and a kernel reading 1,000,000 KiB fetched and 20,000 KiB written moves
    (2 * 1,000,000 + 20,000) * 1024 bytes per launch."""
    run, plan = _fake_run(tmp_path)
    prof = tmp_path / "profiles"
    tpath = prof / "traffic.json"
    recs = bench.ingest_counters(str(run), "chunglu1m_train_bf16", profiles_dir=str(prof),
                                 traffic_path=str(tpath))
    r = recs["fwd_main"]
    assert r["fetch_factor"] == pytest.approx(2.0) and r["write_factor"] == pytest.approx(1.0)
    assert r["bytes_per_launch"] == pytest.approx((2 * 1_000_000 + 20_000) * 1024)
    assert "copy_probe" not in recs
    assert (prof / "chunglu1m_train_bf16.kernel_trace.txt").read_text().count("fwd_main") >= 1
    assert "fetch factor 2.0000" in (prof / "chunglu1m_train_bf16.counters.txt").read_text()
    # read back only for the same sources, plan and node order
    info = dict(plan)
    got = bench.measured_traffic("chunglu1m_train_bf16", "fwd_main", info, "as-generated",
                                 path=str(tpath))
    assert got == pytest.approx(r["bytes_per_launch"])
    info["n_row_sched"] += 1
    assert bench.measured_traffic("chunglu1m_train_bf16", "fwd_main", info, "as-generated",
                                  path=str(tpath)) is None
    assert bench.measured_traffic("chunglu1m_train_bf16", "fwd_main", plan, "rcm",
                                  path=str(tpath)) is None


def test_compulsory_bytes_bound_the_logical_bytes():
    """Every operand row once is never more than one read per gathered edge (E >= N), and
    the dot forward's compulsory bytes are the CSR plus five [N, H, d] / [N, H] arrays."""
    N, E, H, d, b = 1000, 50_000, 8, 32, 2
    for k in ("fwd_main", "bwd_dq_main", "bwd_dkdv_main", "reduce_fwd_main"):
        assert bench.compulsory_bytes(k, N, E, H, d, b) <= bench.algorithmic_bytes(k, N, E, H, d, b)
    assert bench.compulsory_bytes("fwd_main", N, E, H, d, b) == \
        4 * (N + 1) + 4 * E + 4 * N * H * d * b + 4 * N * H
    assert bench.compulsory_bytes("fwd_main", 1_000_000, 50_997_829, 8, 32, 2) == \
        pytest.approx(2.29e9, rel=0.01)


def test_kernel_digests_follow_their_own_sources():
    """A counter record is tied to the source file of its kernel and the shared headers,
    so editing one kernel family's file leaves the other families' records valid."""
    assert bench.kernel_source("fwd_main") == "fwd.hip"
    assert bench.kernel_source("bwd_dkdv_merge") == "bwd.hip"
    assert bench.kernel_source("bwd_gat_cols_main") == "bwd_gat.hip"
    assert bench.kernel_source("bwd_gatv2_rows_main") == "bwd_gatv2.hip"
    assert bench.kernel_source("reduce_bwd_main") == "reduce.hip"
    assert bench.kernel_source("gather_probe_cols") == "probe.hip"
    assert bench.source_digest("fwd_main") == bench.source_digest("fwd_hub_merge")
    assert bench.source_digest("fwd_main") != bench.source_digest("bwd_dq_main")
    csrc = os.path.join(ROOT, "sparse_graph_attention_02_amd", "csrc")
    assert all(os.path.exists(os.path.join(csrc, f)) for _, f in bench.KERNEL_SOURCES)
