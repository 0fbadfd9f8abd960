"""The seeded generators: determinism, CSR conventions and degree statistics."""
import numpy as np
import pytest

import graphgen as gg


def test_same_seed_same_arrays():
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    a = gg.make_graph(w, n=10_000)
    b = gg.make_graph(w, n=10_000)
    assert gg.array_digest(*a) == gg.array_digest(*b)
    fa = gg.make_features(w, n=1000)
    fb = gg.make_features(w, n=1000)
    assert gg.array_digest(*fa) == gg.array_digest(*fb)


@pytest.mark.parametrize("name,n", [("er2k_dot_f32", None), ("chunglu100k_gat_f32", 30_000),
                                    ("rmat21_dot_bf16", 1 << 14)])
def test_csr_conventions(name, n):
    w = gg.WORKLOADS[name]
    ip, ix = gg.make_graph(w, n=n)
    nn = ip.size - 1
    assert ip.dtype == np.int32 and ix.dtype == np.int32 and ip[0] == 0 and ip[-1] == ix.size
    rows = np.repeat(np.arange(nn), np.diff(ip))
    # exactly one self-loop per node
    assert np.array_equal(np.bincount(rows[rows == ix], minlength=nn), np.ones(nn))
    # sources ascending within each row
    same_row = rows[1:] == rows[:-1]
    assert np.all(ix[1:][same_row] >= ix[:-1][same_row])


def test_mean_degree_close_to_nominal():
    w = gg.WORKLOADS["chunglu100k_gat_f32"]
    ip, ix = gg.make_graph(w)
    mean_in = ix.size / w.n - 1.0          # minus the added self-loop
    assert abs(mean_in - 20.0) / 20.0 < 0.02
    assert 7000 < np.diff(ip).max() < 13000   # max in-degree ~10k
    w1 = gg.WORKLOADS["er2k_dot_f32"]
    ip, ix = gg.make_graph(w1)
    assert abs(ix.size / w1.n - 1.0 - 8.0) / 8.0 < 0.02


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -3.0, 65504.0], np.float32)
    b = gg.f32_to_bf16_bits(x)
    back = gg.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even (1 + 2^-6) wins
    assert list(back) == [1.0, 1.0, 1.015625, -3.0, 65536.0]
