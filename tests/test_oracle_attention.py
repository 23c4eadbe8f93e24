"""Oracle attention pinned to closed forms, brute force and torch's SDPA (CPU)."""
import numpy as np
import pytest

import synth
from oracle import (temporal_attn_ref, spatial_attn_ref, spatial_attn_selfrepeat_ref,
                    softmax_rows, bidirectional_temporal_ref, masked_causal_attn_ref)
import pins

TINY = synth.WORKLOADS["tiny_fp32"]


def test_temporal_closed_form_visible_set():
    # before eviction (P_k 0 -> 1 -> 5 -> 9) and after it (wrapped ring)
    assert pins.check_temporal_closed_form(temporal_attn_ref) <= 1e-15
    assert pins.check_temporal_closed_form(temporal_attn_ref, p_max=25, n=8,
                                           writes=(1, 8, 8, 8, 8, 8, 8)) <= 1e-15


def test_temporal_equals_full_recompute_tiny():
    # tiny fp32 shape: 1 + 4 + 4 + 4 + 4 frames, queue full at 9 then evicting
    assert pins.check_temporal_vs_recompute(temporal_attn_ref, TINY) <= 1e-12


def test_temporal_equals_full_recompute_wide():
    shape = dict(B=1, S=2, H=2, d=72, l=8, p_max=25)
    assert pins.check_temporal_vs_recompute(temporal_attn_ref, shape,
                                            writes=(1, 8, 8, 8, 8, 8)) <= 1e-12


def test_temporal_empty_queue_is_causal_sdpa():
    assert pins.check_temporal_empty_queue_is_causal_sdpa(temporal_attn_ref) <= 1e-13


def test_temporal_single_query_is_sdpa():
    assert pins.check_temporal_single_query_is_sdpa(temporal_attn_ref) <= 1e-13


def test_spatial_matches_sdpa():
    assert pins.check_spatial_vs_sdpa(spatial_attn_ref) <= 1e-13


def test_spatial_zero_query_mean():
    assert pins.check_spatial_zero_query(spatial_attn_ref) <= 1e-14


def test_self_repeat_identity():
    g = np.random.default_rng(7)
    B, n, S, H, d, p = 2, 2, 8, 2, 8, 3
    q, k, v = (g.standard_normal((B, n, S, H, d)) for _ in range(3))
    a = spatial_attn_selfrepeat_ref(q, k, v, p, 0.35)
    b = spatial_attn_ref(q, k, v, None, None, [], 0.35, "self")
    assert np.max(np.abs(a - b)) <= 1e-12


def test_spatial_subset_of_queries():
    # evaluating a subset of query tokens gives the same rows as the full call
    g = np.random.default_rng(8)
    B, n, S, H, d = 1, 2, 10, 2, 4
    q, k, v = (g.standard_normal((B, n, S, H, d)) for _ in range(3))
    ks, vs = (g.standard_normal((B, 2, S, H, d)) for _ in range(2))
    full = spatial_attn_ref(q, k, v, ks, vs, [1, 0], 0.5, "prefix")
    sel = [0, 3, 9]
    part = spatial_attn_ref(q[:, :, sel], k, v, ks, vs, [1, 0], 0.5, "prefix")
    assert np.array_equal(full[:, :, sel], part)


def test_softmax_rows_sum_and_shift_invariance():
    g = np.random.default_rng(9)
    z = g.standard_normal((50, 33)) * 30.0
    p = softmax_rows(z)
    assert np.max(np.abs(p.sum(-1) - 1)) <= 1e-12
    # the shift itself rounds z at ~2e-13 (ulp of 1300), so compare at 1e-11
    assert np.max(np.abs(softmax_rows(z + 1234.5) - p)) <= 1e-11
    # huge logits do not overflow
    assert np.all(np.isfinite(softmax_rows(z * 1e6)))


def test_softmax_v_all_ones_gives_ones():
    # V == 1 -> output == 1 whatever the logits (the probe used on the GPU)
    g = np.random.default_rng(10)
    B, n, S, H, d, P = 1, 4, 3, 2, 16, 9
    q, k = (g.standard_normal((B, n, S, H, d)) * 3 for _ in range(2))
    rk = g.standard_normal((B, P, S, H, d)) * 3
    out = temporal_attn_ref(q, k, np.ones((B, n, S, H, d)), rk, np.ones((B, P, S, H, d)),
                            [3, 4, 5, 6, 7, 8, 0, 1, 2], 0.25)
    assert np.max(np.abs(out - 1)) <= 1e-14


def test_bidirectional_matches_sdpa():
    assert pins.check_bidirectional_vs_sdpa(bidirectional_temporal_ref) <= 1e-13


def test_bidirectional_zero_keys_mean():
    assert pins.check_bidirectional_zero_keys(bidirectional_temporal_ref) <= 1e-15


def test_bidirectional_permutation():
    assert pins.check_bidirectional_permutation(bidirectional_temporal_ref) <= 1e-13


def test_bidirectional_last_frame_is_causal():
    assert pins.check_bidirectional_last_frame_is_causal(bidirectional_temporal_ref, temporal_attn_ref) <= 1e-13


def test_bidirectional_brute_force_mask():
    # the explicit-mask form with an all-zero mask, row by row
    g = np.random.default_rng(15)
    B, T, S, H, d = 1, 5, 2, 2, 6
    q, k, v = (g.standard_normal((B, T, S, H, d)) for _ in range(3))
    got = bidirectional_temporal_ref(q, k, v, 0.4)
    for s in range(S):
        for h in range(H):
            ref = masked_causal_attn_ref(q[0, :, s, h], k[0, :, s, h], v[0, :, s, h], np.zeros((T, T)), 0.4)
            assert np.max(np.abs(got[0, :, s, h] - ref)) <= 1e-13
