"""Attention definitions (float64). Test infrastructure only; see oracle/__init__.py.

Layout of every activation tensor: [B][frames][S][H][d] -- batch, frame,
spatial token, head, head dimension. A temporal "row" is one (b, s, h); a
spatial problem is one (b, frame, h).
"""
from __future__ import annotations

import numpy as np

ROW_SUM_TOL = 1e-12


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, max-subtracted, float64.

    Asserts that every row sums to one within 1e-12 (the row-sum property the
    Ca2-VDM notes' CausalAttn equation relies on: Softmax normalises each query
    row over the keys it sees).
    """
    z = np.asarray(z, dtype=np.float64)
    zmax = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    p = e / np.sum(e, axis=-1, keepdims=True)
    err = np.max(np.abs(np.sum(p, axis=-1) - 1.0)) if p.size else 0.0
    assert err <= ROW_SUM_TOL, f"softmax rows do not sum to 1 (err {err})"
    return p


def temporal_attn_ref(q, k_new, v_new, ring_k, ring_v, slot_map, scale):
    """Causal temporal attention over the cached queue plus the new frames.

    Follows the Ca2-VDM notes, key design 1 (causal temporal attention, the
    CausalAttn equation Softmax(QK^T/sqrt(C') + M)V with M_ij = -inf for i < j,
    restated in the abstract page's Formula Representation) and key design 4
    (the temporal KV-cache queue of at most P_max frames).

    For each row (b, s, h) and new query frame i in [0, n): the keys are the
    P_k cached frames in logical order (oldest first, read from ring slots
    ``slot_map``) followed by the new frames 0..n-1; query i sees keys
    j <= P_k + i. Keys it may not see are left out of the softmax, not given a
    large negative logit.

    q, k_new, v_new: [B][n][S][H][d]; ring_k, ring_v: [B][P_slots][S][H][d];
    slot_map: sequence of P_k physical slots. Returns float64 [B][n][S][H][d].
    ``q`` may carry a subset of the tokens/heads of k_new only if k_new, v_new
    and the ring are sliced the same way (rows are independent).

    Pinned by: the K == 0 closed form (mean of the visible values), the
    brute-force masked recompute over the whole sequence, torch's causal SDPA
    when P_k = 0, and unmasked SDPA when n = 1 (tests/test_oracle_attention.py).
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, n, S, H, d = q.shape
    slot_map = [int(s) for s in slot_map]
    P_k = len(slot_map)
    if P_k:
        ck = np.asarray(ring_k, dtype=np.float64)[:, slot_map]
        cv = np.asarray(ring_v, dtype=np.float64)[:, slot_map]
        khat = np.concatenate([ck, k_new], axis=1)
        vhat = np.concatenate([cv, v_new], axis=1)
    else:
        khat, vhat = k_new, v_new
    out = np.empty((B, n, S, H, d), dtype=np.float64)
    for i in range(n):
        visible = P_k + i + 1
        kk = khat[:, :visible]                       # [B][visible][S][H][d]
        vv = vhat[:, :visible]
        z = scale * np.einsum("bshd,bjshd->bshj", q[:, i], kk)
        p = softmax_rows(z)
        out[:, i] = np.einsum("bshj,bjshd->bshd", p, vv)
    return out


def _spatial_keys(k_f, ks, prefix_slots, mode):
    """Key (or value) set of one frame: [B][S_k][H][d]."""
    if mode == "self":
        return k_f
    if mode != "prefix":
        raise ValueError(mode)
    parts = [k_f] + [ks[:, int(s)] for s in prefix_slots]
    return np.concatenate(parts, axis=1)


def spatial_attn_ref(q, k, v, ks, vs, prefix_slots, scale, mode):
    """Prefix-enhanced spatial attention (mode "prefix") or plain spatial
    self-attention (mode "self").

    Follows the Ca2-VDM notes, key design 3 (prefix-enhanced spatial
    attention): a target frame's keys/values are its own S tokens joined along
    the token axis with the tokens of the last P' prefix frames, so the map is
    S x (P'+1)S; and key design 5 (spatial KV-cache holding those frames).
    Mode "self" is the clean-prefix case of key design 3 (self-repeat), whose
    value equals plain self-attention over the frame's own S keys -- checked
    against the literal repeated form by ``spatial_attn_selfrepeat_ref``.

    Key order: own frame first, then the prefix frames oldest to newest (the
    pages do not fix the order; it changes only rounding).

    q: [B][n][S_q][H][d] (S_q may be a subset of tokens); k, v: [B][n][S][H][d];
    ks, vs: [B][P_slots][S][H][d]; prefix_slots: P' physical slots in logical
    order. Returns float64 [B][n][S_q][H][d].

    Pinned by: torch SDPA (no mask) when P' = 0 or mode "self", the Q == 0
    closed form (mean of all value rows), and the self-repeat identity.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if mode == "prefix" and len(prefix_slots):
        ks = np.asarray(ks, dtype=np.float64)
        vs = np.asarray(vs, dtype=np.float64)
    B, n, Sq, H, d = q.shape
    out = np.empty((B, n, Sq, H, d), dtype=np.float64)
    for f in range(n):
        kf = _spatial_keys(k[:, f], ks, prefix_slots, mode)   # [B][Sk][H][d]
        vf = _spatial_keys(v[:, f], vs, prefix_slots, mode)
        for b in range(B):
            qh = q[b, f].transpose(1, 0, 2)          # [H][S_q][d]
            kh = kf[b].transpose(1, 2, 0)            # [H][d][S_k]
            vh = vf[b].transpose(1, 0, 2)            # [H][S_k][d]
            z = scale * np.matmul(qh, kh)            # [H][S_q][S_k]
            p = softmax_rows(z)
            out[b, f] = np.matmul(p, vh).transpose(1, 0, 2)
    return out


def spatial_attn_selfrepeat_ref(q, k, v, p_spatial, scale):
    """The clean-prefix form of key design 3 written out literally: the frame's
    own K/V repeated P'+1 times along the token axis, so the map keeps the
    S x (P'+1)S shape. Used only to check that it equals plain self-attention.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, n, Sq, H, d = q.shape
    out = np.empty((B, n, Sq, H, d), dtype=np.float64)
    for f in range(n):
        kf = np.concatenate([k[:, f]] * (p_spatial + 1), axis=1)
        vf = np.concatenate([v[:, f]] * (p_spatial + 1), axis=1)
        for b in range(B):
            z = scale * np.einsum("shd,thd->hst", q[b, f], kf[b])
            p = softmax_rows(z)
            out[b, f] = np.einsum("hst,thd->shd", p, vf[b])
    return out


def masked_causal_attn_ref(q, k, v, mask_add, scale):
    """Softmax(scale * Q K^T + M) V with an explicit additive mask M (0 or -inf).

    This is the CausalAttn equation of key design 1 taken literally, with M
    given as a matrix. q: [Lq][d], k, v: [Lk][d], mask_add: [Lq][Lk].
    exp(-inf) = 0, so masked keys get zero weight; every row must keep at
    least one finite entry.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = scale * (q @ k.T) + np.asarray(mask_add, dtype=np.float64)
    assert np.all(np.isfinite(z).any(axis=-1)), "a query row sees no key"
    p = softmax_rows(z)
    return p @ v


def full_recompute_temporal_ref(q_chunk, k_seq, v_seq, n0, p_max, scale):
    """Brute-force temporal attention of one chunk over the whole frame sequence.

    The sequence holds frames 0..n0+n-1 (clean frames 0..n0-1, then the n chunk
    frames). Query frame n0+i attends to frames j with w <= j <= n0+i, where
    w = max(0, n0 - P_max): full lower-triangular attention before the queue
    is full (key design 1), and after eviction a window that starts where the
    queue starts -- the same P_max cached frames for every query of the chunk,
    because the queue changes once per autoregressive step (overall framework
    and key design 4 of the Ca2-VDM notes).

    Built as one (n) x (n0+n) additive mask per row and evaluated with
    ``masked_causal_attn_ref``; no ring buffer, no slot map.

    q_chunk: [B][n][S][H][d]; k_seq, v_seq: [B][n0+n][S][H][d].
    """
    q_chunk = np.asarray(q_chunk, dtype=np.float64)
    k_seq = np.asarray(k_seq, dtype=np.float64)
    v_seq = np.asarray(v_seq, dtype=np.float64)
    B, n, S, H, d = q_chunk.shape
    L = k_seq.shape[1]
    assert L == n0 + n
    w = max(0, n0 - p_max)
    M = np.full((n, L), -np.inf)
    for i in range(n):
        qf = n0 + i
        M[i, w:qf + 1] = 0.0
    out = np.empty_like(q_chunk)
    for b in range(B):
        for s in range(S):
            for h in range(H):
                out[b, :, s, h] = masked_causal_attn_ref(
                    q_chunk[b, :, s, h], k_seq[b, :, s, h], v_seq[b, :, s, h], M, scale)
    return out


def bidirectional_temporal_ref(q, k, v, scale):
    """Temporal attention without a cache: every frame attends to every frame.

    This is the recompute baseline the Ca2-VDM pages measure against (the
    abstract page and the notes' speed comparison: existing VDMs attend
    bidirectionally along time, so the conditional frames' K/V depend on the
    noisy frames and are recomputed at every denoising step; OS-Ext extends the
    conditioning and its time grows quadratically with the autoregression
    step). For each row (b, s, h), query frame i in [0, T) attends to all T
    frames with no mask: Softmax(scale * Q K^T) V over the frame axis.

    q, k, v: [B][T][S][H][d]. Returns float64 [B][T][S][H][d].

    Pinned by: permutation equivariance over frames, the last frame equal to
    the causal oracle's last frame, the K == 0 closed form, brute force through
    ``masked_causal_attn_ref`` with an all-zero mask, and torch's unmasked SDPA
    (tests/test_oracle_attention.py).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = scale * np.einsum("btshd,bjshd->bshtj", q, k)
    p = softmax_rows(z)
    return np.einsum("bshtj,bjshd->btshd", p, v)
