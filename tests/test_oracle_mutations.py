"""Planted mistakes in copies of the oracle must fail at least one pin.

Each mutant is the oracle's temporal or spatial definition with one plausible
error (off-by-one mask, wrong slot, dropped scale, transposed operand, a
dropped prefix frame, softmax over the wrong axis). Runs on the CPU only.
"""
import numpy as np
import pytest

import synth
from oracle.attention import softmax_rows
import pins

TINY = synth.WORKLOADS["tiny_fp32"]


def _temporal(visible_fn=lambda P_k, i: P_k + i + 1, slot_shift=0, use_scale=True,
              swap_sh=False):
    def impl(q, k_new, v_new, ring_k, ring_v, slot_map, scale):
        q, k_new, v_new = (np.asarray(x, np.float64) for x in (q, k_new, v_new))
        B, n, S, H, d = q.shape
        P = ring_k.shape[1]
        sm = [(s + slot_shift) % P for s in slot_map]
        P_k = len(sm)
        khat = np.concatenate([np.asarray(ring_k, np.float64)[:, sm], k_new], 1) if P_k else k_new
        vhat = np.concatenate([np.asarray(ring_v, np.float64)[:, sm], v_new], 1) if P_k else v_new
        out = np.empty_like(q)
        for i in range(n):
            vis = max(1, min(visible_fn(P_k, i), P_k + n))
            sc = scale if use_scale else 1.0
            if swap_sh and S == H:
                z = sc * np.einsum("bshd,bjhsd->bshj", q[:, i], khat[:, :vis])
            else:
                z = sc * np.einsum("bshd,bjshd->bshj", q[:, i], khat[:, :vis])
            p = softmax_rows(z)
            out[:, i] = np.einsum("bshj,bjshd->bshd", p, vhat[:, :vis])
        return out
    return impl


def _any_pin_fails(impl):
    checks = [
        lambda: pins.check_temporal_closed_form(impl) > 1e-12,
        lambda: pins.check_temporal_vs_recompute(impl, TINY) > 1e-10,
        lambda: pins.check_temporal_empty_queue_is_causal_sdpa(impl) > 1e-10,
        lambda: pins.check_temporal_single_query_is_sdpa(impl) > 1e-10,
    ]
    return any(c() for c in checks)


def test_oracle_itself_passes_every_temporal_pin():
    assert not _any_pin_fails(_temporal())


@pytest.mark.parametrize("mutant", [
    _temporal(visible_fn=lambda P_k, i: P_k + i),         # query cannot see itself
    _temporal(visible_fn=lambda P_k, i: P_k + i + 2),     # sees the next frame
    _temporal(visible_fn=lambda P_k, i: i + 1),           # ignores the cache
    _temporal(slot_shift=1),                              # wrong ring slot
    _temporal(use_scale=False),                           # dropped 1/sqrt(d)
])
def test_temporal_mutants_are_caught(mutant):
    assert _any_pin_fails(mutant)


def test_transposed_operand_is_caught():
    # S == H so a swapped (token, head) index still runs
    mutant = _temporal(swap_sh=True)

    def check():
        g = np.random.default_rng(0)
        B, n, S, H, d = 1, 3, 3, 3, 4
        q, k, v = (g.standard_normal((B, n, S, H, d)) for _ in range(3))
        got = mutant(q, k, v, np.zeros((B, 1, S, H, d)), np.zeros((B, 1, S, H, d)), [], 0.5)
        perm = (0, 2, 3, 1, 4)
        ref = pins.sdpa64(q.transpose(perm), k.transpose(perm), v.transpose(perm), 0.5, causal=True)
        return float(np.max(np.abs(got.transpose(perm) - ref)))
    assert check() > 1e-6


def _spatial(drop_last_prefix=False, softmax_axis_wrong=False):
    def impl(q, k, v, ks, vs, slots, scale, mode):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        B, n, Sq, H, d = q.shape
        out = np.empty_like(q)
        use = list(slots)[:-1] if (drop_last_prefix and slots) else list(slots)
        for f in range(n):
            if mode == "prefix":
                kk = np.concatenate([k[:, f]] + [ks[:, s] for s in use], 1)
                vv = np.concatenate([v[:, f]] + [vs[:, s] for s in use], 1)
            else:
                kk, vv = k[:, f], v[:, f]
            for b in range(B):
                z = scale * np.einsum("shd,thd->hst", q[b, f], kk[b])
                if softmax_axis_wrong:
                    e = np.exp(z - z.max(1, keepdims=True))
                    p = e / e.sum(1, keepdims=True)
                else:
                    p = softmax_rows(z)
                out[b, f] = np.einsum("hst,thd->shd", p, vv[b])
        return out
    return impl


@pytest.mark.parametrize("mutant", [_spatial(drop_last_prefix=True), _spatial(softmax_axis_wrong=True)])
def test_spatial_mutants_are_caught(mutant):
    assert pins.check_spatial_vs_sdpa(mutant) > 1e-6 or pins.check_spatial_zero_query(mutant) > 1e-6


def test_spatial_oracle_passes():
    from oracle import spatial_attn_ref
    assert pins.check_spatial_vs_sdpa(_spatial()) <= 1e-13
    assert pins.check_spatial_vs_sdpa(spatial_attn_ref) <= 1e-13


def _bidir(mask_causal=False, use_scale=True, swap_qk=False, axis_bug=False):
    def impl(q, k, v, scale):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        sc = scale if use_scale else 1.0
        a, b = (k, q) if swap_qk else (q, k)
        z = sc * np.einsum("btshd,bjshd->bshtj", a, b)
        T = q.shape[1]
        if mask_causal:
            z = z + np.triu(np.full((T, T), -np.inf), 1)
        if axis_bug:
            p = np.exp(z - z.max(axis=-2, keepdims=True))
            p = p / p.sum(axis=-2, keepdims=True)
        else:
            p = softmax_rows(z)
        return np.einsum("bshtj,bjshd->btshd", p, v)
    return impl


def _bidir_pin_fails(impl):
    from oracle import temporal_attn_ref
    checks = [
        lambda: pins.check_bidirectional_vs_sdpa(impl) > 1e-10,
        lambda: pins.check_bidirectional_zero_keys(impl) > 1e-12,
        lambda: pins.check_bidirectional_permutation(impl) > 1e-10,
        lambda: pins.check_bidirectional_last_frame_is_causal(impl, temporal_attn_ref) > 1e-10,
    ]
    return any(c() for c in checks)


def test_bidirectional_oracle_passes_every_pin():
    assert not _bidir_pin_fails(_bidir())


@pytest.mark.parametrize("mutant", [
    _bidir(mask_causal=True),      # causal mask where none belongs
    _bidir(use_scale=False),       # dropped scale
    _bidir(swap_qk=True),          # Q and K swapped (transposed logits)
    _bidir(axis_bug=True),         # softmax over the query axis
], ids=["causal_mask", "no_scale", "swap_qk", "softmax_axis"])
def test_bidirectional_mutants_fail_a_pin(mutant):
    assert _bidir_pin_fails(mutant)
