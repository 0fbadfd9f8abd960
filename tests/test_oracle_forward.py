"""Pins of the fp64 oracle's forward against things other than itself.

Each test is chosen so that a plausible mistake in the oracle (a wrong index, a dropped
parallel edge, a missing max-shift, a transposed operand, a wrong head split, the LeakyReLU
branch swapped) fails at least one of them:

* hand-derived closed forms (tests/golden/worked_example.json),
* dense masked attention written as N x N matrix algebra (brute force, multiplicities),
* torch's fp64 scaled_dot_product_attention with a boolean / additive log-count mask,
* scipy's logsumexp for the row statistic,
* GAT closed forms where LeakyReLU is linear on the whole row,
* invariants: weights sum to 1, single-neighbour rows, uniform scores, permutations.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import graphgen as gg
from oracle import attention as A

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _load_golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    arr = lambda key: np.array(g[key], dtype=np.float64)
    return g, arr


def test_worked_example_values_are_the_closed_forms(golden_dir):
    g, _ = _load_golden(golden_dir)
    ln3 = math.log(3.0)
    ex = g["expected"]
    assert g["k"][1][0][0] == ln3
    assert ex["lse"][0][0] == math.log(4.0)
    assert ex["lse"][2][0] == ln3
    assert ex["out"][2][0][1] == -2.0 / 3.0
    assert ex["dq"][0][0][0] == 0.75 * ln3
    assert ex["dq"][2][0][0] == -1.0 + 2.0 * ln3


def test_worked_example_forward(golden_dir):
    g, arr = _load_golden(golden_dir)
    ip = np.array(g["indptr"], np.int32)
    ix = np.array(g["indices"], np.int32)
    out, lse = A.forward(ip, ix, arr("q"), arr("k"), arr("v"), "dot", g["scale"])
    exp_out = np.array(g["expected"]["out"])
    exp_lse = np.array([[float(x[0])] for x in g["expected"]["lse"]])
    np.testing.assert_allclose(out, exp_out, rtol=0, atol=1e-14)
    assert np.isneginf(lse[3, 0])
    np.testing.assert_allclose(lse[:3], exp_lse[:3], rtol=0, atol=1e-14)
    # the single-neighbour row is exact, not just close
    assert np.array_equal(out[1], arr("v")[0])


def _dense_counts(indptr, indices, n):
    c = np.zeros((n, n))
    for i in range(n):
        for j in indices[indptr[i]:indptr[i + 1]]:
            c[i, j] += 1
    return c


def _dense_attention(c, S, V):
    """Dense masked attention with multiplicities: rows = destinations.
    S [H, N, N] scores, V [N, H, d], c [N, N] edge counts."""
    H = S.shape[0]
    n = c.shape[0]
    out = np.zeros((n, H, V.shape[2]))
    lse = np.full((n, H), -np.inf)
    for h in range(H):
        Sm = np.where(c > 0, S[h], -np.inf)
        rmax = Sm.max(axis=1)
        has = c.sum(axis=1) > 0
        W = np.zeros_like(Sm)
        W[has] = c[has] * np.exp(Sm[has] - rmax[has, None])
        Z = W.sum(axis=1)
        out[has, h, :] = (W[has] @ V[:, h, :]) / Z[has, None]
        lse[has, h] = rmax[has] + np.log(Z[has])
    return out, lse


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dot_matches_dense_bruteforce_with_multiplicity(seed):
    rng = np.random.default_rng(seed)
    n, H, d = 23, 3, 5
    src = np.r_[rng.integers(0, n, 200), 3, 3, 3]     # three parallel 3 -> 5 edges
    dst = np.r_[rng.integers(0, n, 200), 5, 5, 5]
    keep_empty = 7                                      # row 7 gets no edges
    ip, ix = gg.csr_from_edges(n, src[dst != keep_empty], dst[dst != keep_empty])
    assert ip[keep_empty + 1] == ip[keep_empty]
    q = rng.standard_normal((n, H, d))
    k = rng.standard_normal((n, H, d))
    v = rng.standard_normal((n, H, d))
    scale = 0.37
    out, lse = A.forward(ip, ix, q, k, v, "dot", scale)
    c = _dense_counts(ip, ix, n)
    assert c[5, 3] >= 3
    S = scale * np.einsum("ihc,jhc->hij", q, k)
    ref, ref_lse = _dense_attention(c, S, v)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1])
def test_gat_matches_dense_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n, H, d = 19, 4, 3
    ip, ix = gg.random_multigraph(n, 60, rng)
    s = rng.standard_normal((n, H))
    t = rng.standard_normal((n, H))
    v = rng.standard_normal((n, H, d))
    out, lse = A.forward(ip, ix, s, t, v, "gat", 1.0, 0.2)
    c = _dense_counts(ip, ix, n)
    x = s.T[:, :, None] + t.T[:, None, :]          # [H, i, j]
    S = np.maximum(x, 0) + 0.2 * np.minimum(x, 0)
    ref, ref_lse = _dense_attention(c, S, v)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_dot_matches_torch_sdpa_on_er2k():
    """torch's fp64 scaled_dot_product_attention with a boolean adjacency mask on the
    2,000-node Erdos-Renyi graph (simple graph, self-loops, one head, d = 32)."""
    w = gg.WORKLOADS["er2k_dot_f32"]
    ip, ix = gg.make_graph(w)
    q, k, v = gg.make_features(w)
    out, lse = A.forward(ip, ix, q, k, v, "dot", np.float32(1 / np.sqrt(32)))
    n = w.n
    mask = torch.zeros(n, n, dtype=torch.bool)
    rows = torch.from_numpy(np.repeat(np.arange(n), np.diff(ip)))
    mask[rows, torch.from_numpy(ix.astype(np.int64))] = True
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2).contiguous()
    tk = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).contiguous()
    tv = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=float(np.float32(1 / np.sqrt(32))))
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_multigraph_matches_torch_sdpa_with_log_count_mask():
    rng = np.random.default_rng(7)
    n, H, d = 40, 2, 8
    ip, ix = gg.random_multigraph(n, 900, rng)  # dense enough for many parallel edges
    c = _dense_counts(ip, ix, n)
    assert c.max() >= 2
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    out, _ = A.forward(ip, ix, q, k, v, "dot", None)
    add = torch.from_numpy(np.where(c > 0, np.log(np.maximum(c, 1)), -np.inf))
    T = lambda x: torch.from_numpy(x).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(T(q), T(k), T(v), attn_mask=add)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(3)
    n, H, d = 30, 2, 4
    ip, ix = gg.random_multigraph(n, 200, rng)
    q, k, v = (rng.standard_normal((n, H, d)) * 4 for _ in range(3))
    _, lse = A.forward(ip, ix, q, k, v, "dot", 1.0)
    for i in range(n):
        J = ix[ip[i]:ip[i + 1]]
        e = np.einsum("hc,khc->kh", q[i], k[J])
        np.testing.assert_allclose(lse[i], logsumexp(e, axis=0), rtol=1e-13)


def test_gat_closed_form_positive_branch():
    """s_i + min_j t_j >= 0 on a row: LeakyReLU is the identity, s_i cancels, and the row
    is softmax(t_j) weighting."""
    rng = np.random.default_rng(11)
    n, H, d = 25, 3, 4
    ip, ix = gg.random_multigraph(n, 120, rng)
    t = rng.standard_normal((n, H))
    s = np.full((n, H), 50.0)
    v = rng.standard_normal((n, H, d))
    out, _ = A.forward(ip, ix, s, t, v, "gat", 1.0, 0.2)
    for i in range(n):
        J = ix[ip[i]:ip[i + 1]]
        w = np.exp(t[J] - t[J].max(0))
        ref = np.einsum("kh,khc->hc", w / w.sum(0), v[J])
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-13)


def test_gat_closed_form_negative_branch():
    """s_i + max_j t_j < 0: every score is neg_slope * (s_i + t_j); weights are
    softmax(neg_slope * t_j) (s_i cancels again)."""
    rng = np.random.default_rng(12)
    n, H, d = 25, 2, 3
    ip, ix = gg.random_multigraph(n, 120, rng)
    t = rng.standard_normal((n, H))
    s = np.full((n, H), -50.0)
    v = rng.standard_normal((n, H, d))
    a = 0.2
    out, _ = A.forward(ip, ix, s, t, v, "gat", 1.0, a)
    for i in range(n):
        J = ix[ip[i]:ip[i + 1]]
        z = a * t[J]
        w = np.exp(z - z.max(0))
        ref = np.einsum("kh,khc->hc", w / w.sum(0), v[J])
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-13)


def test_weights_sum_to_one_and_are_positive():
    rng = np.random.default_rng(5)
    n, H, d = 50, 4, 8
    ip, ix = gg.random_multigraph(n, 400, rng)
    q, k = (rng.standard_normal((n, H, d)) * 3 for _ in range(2))
    for i in range(n):
        alpha, _ = A.row_softmax(A.row_scores(i, ip, ix, q, k, "dot", 1.0))
        assert np.all(alpha > 0)
        np.testing.assert_allclose(alpha.sum(axis=0), 1.0, rtol=0, atol=1e-15)


def test_single_neighbour_rows_return_v_exactly():
    rng = np.random.default_rng(6)
    n, H, d = 40, 2, 16
    src = rng.integers(0, n, n)
    ip, ix = gg.csr_from_edges(n, src, np.arange(n))
    q, k, v = (rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(3))
    out, lse = A.forward(ip, ix, q, k, v, "dot", None)
    assert np.array_equal(out, v[src].astype(np.float64))
    np.testing.assert_allclose(lse, np.einsum("ihc,ihc->ih", q.astype(np.float64),
                                              k[src].astype(np.float64)) / 4.0, rtol=1e-14)


def test_uniform_scores_give_neighbour_mean():
    rng = np.random.default_rng(8)
    n, H, d = 60, 2, 6
    ip, ix = gg.random_multigraph(n, 500, rng)
    q = np.zeros((n, H, d))
    k, v = (rng.standard_normal((n, H, d)) for _ in range(2))
    out, lse = A.forward(ip, ix, q, k, v, "dot", None)
    s = np.zeros((n, H))
    out_g, _ = A.forward(ip, ix, s, s, v, "gat", 1.0, 0.2)
    for i in range(n):
        J = ix[ip[i]:ip[i + 1]]
        np.testing.assert_allclose(out[i], v[J].mean(axis=0), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(out_g[i], v[J].mean(axis=0), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[i], np.log(J.size), rtol=1e-14)


def test_neighbour_permutation_invariance():
    rng = np.random.default_rng(9)
    n, H, d = 45, 3, 5
    ip, ix = gg.random_multigraph(n, 400, rng)
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    out, lse = A.forward(ip, ix, q, k, v, "dot", None)
    ix2 = ix.copy()
    for i in range(n):
        seg = ix2[ip[i]:ip[i + 1]]
        ix2[ip[i]:ip[i + 1]] = seg[rng.permutation(seg.size)]
    out2, lse2 = A.forward(ip, ix2, q, k, v, "dot", None)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14, atol=1e-14)


def test_forward_rows_subset_matches_full():
    rng = np.random.default_rng(10)
    n, H, d = 70, 2, 4
    ip, ix = gg.random_multigraph(n, 500, rng)
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    out, lse = A.forward(ip, ix, q, k, v, "dot", None)
    rows = rng.choice(n, 15, replace=False)
    o2, l2 = A.forward_rows(ip, ix, q, k, v, rows, "dot", None)
    assert np.array_equal(o2, out[rows]) and np.array_equal(l2, lse[rows])


def test_bf16_inputs_are_widened_exactly():
    x = np.array([1.0, -2.5, 3.140625, 1e-3], dtype=np.float32)
    bits = gg.f32_to_bf16_bits(x)
    w = A.widen(bits)
    # bf16 keeps 8 significant bits: exact for the first three, RNE for the last
    assert list(w[:3]) == [1.0, -2.5, 3.140625]
    assert abs(w[3] - 1e-3) <= 2 ** -9 * 1e-3 and w.dtype == np.float64


@pytest.mark.parametrize("max_chunk", [None, 1, 3, 1000])
@pytest.mark.parametrize("score", ["dot", "gat"])
def test_online_chunked_equals_two_pass(score, max_chunk):
    """The streaming form (running max, sum and accumulator per edge; rows cut into chunks
    at random boundaries whose states merge in order) equals the two-pass definition to
    1e-13: one chunk per row (max_chunk 1000: pure online), one edge per chunk, and mixes."""
    rng = np.random.default_rng(5 if score == "dot" else 6)
    n, H, d = 150, 3, 8
    ip, ix = gg.random_multigraph(n, 1800, rng, hub_rows=(4, 40), hub_deg=300)
    if score == "dot":
        a, b = (rng.standard_normal((n, H, d)) * 1.5 for _ in range(2))
    else:
        a, b = (rng.standard_normal((n, H)) * 2 for _ in range(2))
    v = rng.standard_normal((n, H, d))
    ro, rl = A.forward(ip, ix, a, b, v, score)
    co, cl = A.forward_online_chunked(ip, ix, a, b, v, np.random.default_rng(9), score,
                                      max_chunk=max_chunk)
    assert np.array_equal(np.isneginf(cl), np.isneginf(rl))
    fin = ~np.isneginf(rl)
    assert np.allclose(cl[fin], rl[fin], rtol=1e-13, atol=1e-13)
    assert np.allclose(co, ro, rtol=1e-13, atol=1e-13)


def test_online_chunked_keeps_empty_rows_and_large_scores():
    """Rows without neighbours stay (0, -inf); scores in the hundreds (exp would overflow
    without the running max) still match."""
    ip = np.array([0, 0, 3, 3, 5])
    ix = np.array([1, 2, 3, 0, 0])
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((4, 2, 4)) * 12, rng.standard_normal((4, 2, 4)) * 12
    v = rng.standard_normal((4, 2, 4))
    ro, rl = A.forward(ip, ix, q, k, v, "dot", scale=1.0)
    assert np.abs(rl[np.isfinite(rl)]).max() > 100
    co, cl = A.forward_online_chunked(ip, ix, q, k, v, rng, "dot", scale=1.0, max_chunk=1)
    assert np.all(co[[0, 2]] == 0) and np.all(np.isneginf(cl[[0, 2]]))
    assert np.allclose(co, ro, rtol=1e-13, atol=1e-13) and np.allclose(cl[[1, 3]], rl[[1, 3]],
                                                                       rtol=1e-13)
