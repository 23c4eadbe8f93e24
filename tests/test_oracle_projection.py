"""QKV projection oracle pinned by one-hot inputs, brute force and linearity."""
import numpy as np

from oracle import qkv_proj_ref


def test_one_hot_rows_pick_weight_columns():
    g = np.random.default_rng(0)
    C = 6
    w = g.standard_normal((3 * C, C))
    x = np.eye(C)[[3, 0, 5, 5]]
    q, k, v = qkv_proj_ref(x, w)
    for r, col in enumerate([3, 0, 5, 5]):
        assert np.array_equal(q[r], w[:C, col])
        assert np.array_equal(k[r], w[C:2 * C, col])
        assert np.array_equal(v[r], w[2 * C:, col])


def test_brute_force_triple_loop():
    g = np.random.default_rng(1)
    M, Cin, C = 5, 7, 3
    x = g.standard_normal((M, Cin))
    w = g.standard_normal((3 * C, Cin))
    y = np.zeros((M, 3 * C))
    for i in range(M):
        for j in range(3 * C):
            for kk in range(Cin):
                y[i, j] += x[i, kk] * w[j, kk]
    q, k, v = qkv_proj_ref(x, w)
    assert np.max(np.abs(np.concatenate([q, k, v], 1) - y)) <= 1e-12


def test_linearity():
    g = np.random.default_rng(2)
    x1, x2 = g.standard_normal((2, 4, 8))
    w = g.standard_normal((12, 8))
    a = np.concatenate(qkv_proj_ref(2 * x1 - 3 * x2, w), 1)
    b = 2 * np.concatenate(qkv_proj_ref(x1, w), 1) - 3 * np.concatenate(qkv_proj_ref(x2, w), 1)
    assert np.max(np.abs(a - b)) <= 1e-12
