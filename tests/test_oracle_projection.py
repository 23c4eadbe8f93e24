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


# --- projection with the cyclic TPE row --------------------------------------
import pytest  # noqa: E402

import pins  # noqa: E402
from oracle import qkv_proj_tpe_ref  # noqa: E402
from oracle.projection import qkv_proj_ref as _plain  # noqa: E402


def test_tpe_zero_input_gives_table_rows():
    assert pins.check_tpe_proj_zero_input(qkv_proj_tpe_ref) == 0.0


def test_tpe_equals_projecting_embedded_tokens():
    assert pins.check_tpe_proj_distributive(qkv_proj_tpe_ref) <= 1e-12


def _tpe_mutant(kind):
    def impl(x, w, rows, first, n, S):
        x = np.asarray(x, np.float64)
        y = np.concatenate(_plain(x, w), 1)
        L = rows.shape[0]
        for r in range(x.shape[0]):
            f = (r // S) % n
            if kind == "no_add":
                continue
            if kind == "off_by_one":
                i = (first + f + 1) % L
            elif kind == "no_wrap":
                i = min(first + f, L - 1)
            elif kind == "frame_ignores_batch":
                i = (first + min(r // S, n - 1)) % L
            elif kind == "token_index":
                i = (first + (r % S)) % L
            else:
                i = (first + f) % L
            y[r] += rows[i] if kind != "k_only" else np.concatenate([0 * rows[i][:y.shape[1] // 3],
                                                                     rows[i][y.shape[1] // 3:]])
        C = y.shape[1] // 3
        return y[:, :C], y[:, C:2 * C], y[:, 2 * C:]
    return impl


@pytest.mark.parametrize("kind", ["no_add", "off_by_one", "no_wrap", "frame_ignores_batch", "token_index",
                                  "k_only"])
def test_tpe_mutants_fail_a_pin(kind):
    m = _tpe_mutant(kind)
    assert pins.check_tpe_proj_zero_input(m) > 1e-9 or pins.check_tpe_proj_distributive(m) > 1e-9


def test_tpe_mutant_harness_passes_unmutated():
    m = _tpe_mutant("none")
    assert pins.check_tpe_proj_zero_input(m) == 0.0 and pins.check_tpe_proj_distributive(m) <= 1e-12
