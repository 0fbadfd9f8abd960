"""Pins of the oracle's GATv2 score (the textbook definition: e = a . LeakyReLU(xd_i + xs_j),
message xs_j) and its backward."""
import numpy as np
import pytest
import torch

import graphgen as gg
from oracle import attention as A


def _inputs(seed, n, m, H=2, d=3):
    rng = np.random.default_rng(seed)
    ip, ix = gg.random_multigraph(n, m, rng)
    xd, xs, do = (rng.standard_normal((n, H, d)) for _ in range(3))
    a = rng.standard_normal((H, d))
    return ip, ix, xd, xs, a, do


def _dense(ip, ix, xd, xs, a, scale, slope, requires_grad=False):
    n, H, d = xd.shape
    c = np.zeros((n, n))
    np.add.at(c, (np.repeat(np.arange(n), np.diff(ip)), ix), 1.0)
    add = torch.from_numpy(np.where(c > 0, np.log(np.maximum(c, 1)), -np.inf))
    txd = torch.from_numpy(xd.copy()).requires_grad_(requires_grad)
    txs = torch.from_numpy(xs.copy()).requires_grad_(requires_grad)
    ta = torch.from_numpy(a.copy()).requires_grad_(requires_grad)
    z = txd[:, None] + txs[None, :]                                  # [i, j, H, d]
    e = scale * (torch.nn.functional.leaky_relu(z, slope) * ta).sum(-1)   # [i, j, H]
    e = e.permute(2, 0, 1) + add                                    # [H, i, j]
    has = torch.from_numpy(c.sum(1) > 0)
    P = torch.softmax(e[:, has], dim=-1)
    out = torch.zeros(H, n, d, dtype=torch.float64)
    out[:, has] = torch.matmul(P, txs.permute(1, 0, 2).contiguous())
    return out.permute(1, 0, 2), (txd, txs, ta)


@pytest.mark.parametrize("seed", [0, 1])
def test_gatv2_forward_matches_dense_torch(seed):
    ip, ix, xd, xs, a, _ = _inputs(seed, 25, 300, H=3, d=4)
    out, lse = A.forward_gatv2(ip, ix, xd, xs, a, 0.7, 0.1)
    ref, _ = _dense(ip, ix, xd, xs, a, 0.7, 0.1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_gatv2_closed_forms():
    ip, ix, xd, xs, a, _ = _inputs(3, 40, 400, H=2, d=5)
    # a = 0: uniform weights, the mean of the neighbour messages
    out, lse = A.forward_gatv2(ip, ix, xd, xs, np.zeros_like(a))
    for i in range(40):
        J = ix[ip[i]:ip[i + 1]]
        np.testing.assert_allclose(out[i], xs[J].mean(axis=0), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[i], np.log(J.size), rtol=1e-14)
    # every z >= 0: e = a.xd_i + a.xs_j, so the row softmax ignores xd and is softmax(a.xs_j)
    xd_big = xd + 100.0
    out, _ = A.forward_gatv2(ip, ix, xd_big, xs, a)
    for i in range(40):
        J = ix[ip[i]:ip[i + 1]]
        e = np.einsum("hc,khc->kh", a, xs[J])
        w = np.exp(e - e.max(0))
        ref = np.einsum("kh,khc->hc", w / w.sum(0), xs[J])
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-13)


def test_gatv2_backward_matches_torch_autograd():
    ip, ix, xd, xs, a, do = _inputs(5, 20, 200, H=2, d=3)
    dst = np.repeat(np.arange(20), np.diff(ip))
    ip, ix = gg.csr_from_edges(20, ix[dst != 4], dst[dst != 4])      # row 4 empty
    gxd, gxs, ga = A.backward_gatv2(ip, ix, xd, xs, a, do, 1.3, 0.15)
    out, (txd, txs, ta) = _dense(ip, ix, xd, xs, a, 1.3, 0.15, requires_grad=True)
    (out * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(gxd, txd.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gxs, txs.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ga, ta.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_gatv2_backward_finite_differences():
    ip, ix, xd, xs, a, do = _inputs(6, 8, 25, H=2, d=2)
    gxd, gxs, ga = A.backward_gatv2(ip, ix, xd, xs, a, do, 0.9, 0.2)

    def loss(xd_, xs_, a_):
        out, _ = A.forward_gatv2(ip, ix, xd_, xs_, a_, 0.9, 0.2)
        return float((out * do).sum())

    h = 1e-6
    for name, x, g in (("xd", xd, gxd), ("xs", xs, gxs), ("a", a, ga)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            p_ = {"xd": xd, "xs": xs, "a": a}; m_ = dict(p_)
            xp = x.copy(); xp[idx] += h; p_[name] = xp
            xm = x.copy(); xm[idx] -= h; m_[name] = xm
            num[idx] = (loss(p_["xd"], p_["xs"], p_["a"]) - loss(m_["xd"], m_["xs"], m_["a"])) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_gatv2_sampled_forms_agree():
    ip, ix, xd, xs, a, do = _inputs(7, 60, 700, H=2, d=4)
    gxd, gxs, ga = A.backward_gatv2(ip, ix, xd, xs, a, do)
    sel = np.random.default_rng(0).choice(60, 12, replace=False)
    rxd, _ = A.grad_gatv2_rows(ip, ix, xd, xs, a, do, sel)
    np.testing.assert_allclose(rxd, gxd[sel], rtol=1e-12, atol=1e-13)
    _, da_all = A.grad_gatv2_rows(ip, ix, xd, xs, a, do, np.arange(60))
    np.testing.assert_allclose(da_all, ga, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A.grad_gatv2_cols(ip, ix, xd, xs, a, do, sel), gxs[sel],
                               rtol=1e-12, atol=1e-13)


def test_train_step_rows_gatv2_is_the_plain_step():
    ip, ix, xd, xs, a, do = _inputs(11, 30, 250, H=2, d=4)
    out, lse = A.forward_gatv2(ip, ix, xd, xs, a, 0.8, 0.15)
    dxd, dxs, da = A.backward_gatv2(ip, ix, xd, xs, a, do, 0.8, 0.15)
    o2, l2, dxd2, cols, dxs2, da2 = A.train_step_rows_gatv2(ip, ix, xd, xs, a, do,
                                                           np.arange(30), 0.8, 0.15)
    np.testing.assert_allclose(o2, out, atol=1e-13)
    np.testing.assert_allclose(l2, lse, atol=1e-13)
    np.testing.assert_allclose(dxd2, dxd, atol=1e-12)
    full = np.zeros_like(dxs)
    full[cols] = dxs2
    np.testing.assert_allclose(full, dxs, atol=1e-12)
    np.testing.assert_allclose(da2, da, atol=1e-12)
    # a subset of rows gives those rows' shares
    rows = np.array([2, 7, 19])
    o3, _, dxd3, _, _, _ = A.train_step_rows_gatv2(ip, ix, xd, xs, a, do, rows, 0.8, 0.15)
    np.testing.assert_allclose(o3, out[rows], atol=1e-13)
    np.testing.assert_allclose(dxd3, dxd[rows], atol=1e-12)


@pytest.mark.parametrize("slope", [0.2, 1.7])
def test_gatv2_row_and_column_passes_in_blocks_are_the_plain_step(slope):
    """The GATv2 halves run over random blocks of rows and columns reproduce forward_gatv2
    and backward_gatv2 (pinned above by dense autograd and finite differences); the
    blocks' dattn shares sum to dattn."""
    rng = np.random.default_rng(41)
    n, H, d = 60, 2, 4
    ip, ix = gg.random_multigraph(n, 700, rng, self_loops=False, hub_rows=(5,), hub_deg=90)
    dst = np.repeat(np.arange(n), np.diff(ip))
    keep = (dst != 7) & (ix != 13)                      # row 7 and column 13 empty
    ip, ix = gg.csr_from_edges(n, ix[keep], dst[keep])
    xd, xs, do = (rng.standard_normal((n, H, d)) for _ in range(3))
    attn = rng.standard_normal((H, d))
    fo, fl = A.forward_gatv2(ip, ix, xd, xs, attn, 0.8, slope)
    dxd0, dxs0, da0 = A.backward_gatv2(ip, ix, xd, xs, attn, do, 0.8, slope)
    ea, ed = np.full((ix.size, H), np.nan), np.full((ix.size, H), np.nan)
    da = np.zeros((H, d))
    cuts = np.unique(np.r_[0, rng.choice(n, 5), n])
    for r0, r1 in zip(cuts[:-1], cuts[1:]):
        out, lse, dxd, a, e, dap = A.row_pass_gatv2(ip, ix, xd, xs, attn, do,
                                                   np.arange(r0, r1), 0.8, slope)
        np.testing.assert_allclose(out, fo[r0:r1], rtol=1e-13, atol=1e-14)
        fin = ~np.isneginf(fl[r0:r1])
        np.testing.assert_allclose(lse[fin], fl[r0:r1][fin], rtol=1e-13)
        np.testing.assert_allclose(dxd, dxd0[r0:r1], rtol=1e-12, atol=1e-12)
        ea[ip[r0]:ip[r1]], ed[ip[r0]:ip[r1]] = a, e
        da += dap
    assert not np.isnan(ea).any() and not np.isnan(ed).any()
    np.testing.assert_allclose(da, da0, rtol=1e-12, atol=1e-12)
    order, col_start, edge_row = A.transpose_order(ip, ix)
    for c0, c1 in ((0, 13), (13, 14), (14, n)):
        dxs = A.column_pass_gatv2(xd, xs, attn, do, ea, ed, order, col_start, edge_row,
                                  np.arange(c0, c1), 0.8, slope)
        np.testing.assert_allclose(dxs, dxs0[c0:c1], rtol=1e-12, atol=1e-12)
    assert np.all(dxs0[13] == 0) and np.all(dxd0[7] == 0)
