"""Checks that pin the oracle to what the pages and the mathematics fix.

Each check takes the implementation under test as an argument, so the same
check runs on the oracle (tests/test_oracle_*.py) and on deliberately broken
copies of it (tests/test_oracle_mutations.py), which it must reject.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import synth


def sdpa64(q, k, v, scale, causal=False):
    """torch's CPU scaled_dot_product_attention in float64.
    q: [..., Lq, d]; k, v: [..., Lk, d]."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v))
    return F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale).numpy()


# ---------------------------------------------------------------------------
# temporal attention
# ---------------------------------------------------------------------------
def check_temporal_closed_form(temporal_impl, p_max=9, n=4, writes=(1, 4, 4, 4), S=3, H=2):
    """K == 0 makes every visible logit equal, so output i is the mean of the
    visible values. With one-hot frame codes as values the output spells out
    exactly which frames query i sees and how many. Checked after each write,
    so both the growing queue and the post-eviction (wrapped ring) states are
    covered. Returns the max error."""
    from oracle import TemporalQueue
    d = p_max + n            # one code dimension per logical key position
    B = 1
    q_ = TemporalQueue(p_max)
    ring_k = np.zeros((B, p_max, S, H, d))
    ring_v = np.zeros((B, p_max, S, H, d))
    frame = 0
    worst = 0.0
    for w in writes:
        # state before this write: P_k cached frames, logical j -> slot
        slots = q_.slot_map()
        P_k = len(slots)
        # values of the cached frame at logical j: one-hot e_j; new frame i: e_{P_k+i}
        for j, s in enumerate(slots):
            ring_v[:, s] = 0.0
            ring_v[:, s, :, :, j] = 1.0
        k_new = np.zeros((B, n, S, H, d))
        v_new = np.zeros((B, n, S, H, d))
        for i in range(n):
            v_new[:, i, :, :, P_k + i] = 1.0
        q = np.random.default_rng(frame).standard_normal((B, n, S, H, d))
        out = temporal_impl(q, k_new, v_new, ring_k, ring_v, slots, 0.37)
        for i in range(n):
            expect = np.zeros(d)
            expect[:P_k + i + 1] = 1.0 / (P_k + i + 1)
            worst = max(worst, float(np.max(np.abs(out[:, i] - expect))))
        # write w frames (their values are rewritten before the next call)
        q_.write(range(frame, frame + w))
        frame += w
    return worst


def check_temporal_vs_recompute(temporal_impl, shape, seed=3, writes=(1, 4, 4, 4, 4)):
    """Cached-prefix attention equals brute-force masked attention over the
    whole frame sequence, before and after eviction. Returns max abs error."""
    from oracle import TemporalQueue, full_recompute_temporal_ref
    B, S, H, d, n, p_max = (shape[k] for k in ("B", "S", "H", "d", "l", "p_max"))
    scale = 1.0 / np.sqrt(d)
    queue = TemporalQueue(p_max)
    ring_k = np.zeros((B, p_max, S, H, d))
    ring_v = np.zeros((B, p_max, S, H, d))
    frame = 0
    worst = 0.0
    for step, w in enumerate(writes):
        if frame > 0:
            q = synth.step_tensor(seed, "q", step, 1, B, n, S, H, d)
            k = synth.step_tensor(seed, "k", step, 1, B, n, S, H, d)
            v = synth.step_tensor(seed, "v", step, 1, B, n, S, H, d)
            got = temporal_impl(q, k, v, ring_k, ring_v, queue.slot_map(), scale)
            kseq = np.concatenate([synth.frames_tensor(seed, "kt", range(frame), B, S, H, d), k], 1)
            vseq = np.concatenate([synth.frames_tensor(seed, "vt", range(frame), B, S, H, d), v], 1)
            ref = full_recompute_temporal_ref(q, kseq, vseq, frame, p_max, scale)
            worst = max(worst, float(np.max(np.abs(got - ref))))
        frames = list(range(frame, frame + w))
        slots = queue.write(frames)
        kt = synth.frames_tensor(seed, "kt", frames, B, S, H, d)
        vt = synth.frames_tensor(seed, "vt", frames, B, S, H, d)
        for i, s in enumerate(slots):
            ring_k[:, s] = kt[:, i]
            ring_v[:, s] = vt[:, i]
        frame += w
    return worst


def check_temporal_empty_queue_is_causal_sdpa(temporal_impl, B=2, n=5, S=3, H=2, d=8, seed=1):
    """P_k = 0: causal attention over the n new frames, i.e. torch's causal SDPA."""
    g = np.random.default_rng(seed)
    q, k, v = (g.standard_normal((B, n, S, H, d)) for _ in range(3))
    scale = 0.29
    got = temporal_impl(q, k, v, np.zeros((B, 1, S, H, d)), np.zeros((B, 1, S, H, d)), [], scale)
    # rows (b, s, h) -> SDPA batch; frames -> sequence
    perm = (0, 2, 3, 1, 4)
    ref = sdpa64(q.transpose(perm), k.transpose(perm), v.transpose(perm), scale, causal=True)
    return float(np.max(np.abs(got.transpose(perm) - ref)))


def check_temporal_single_query_is_sdpa(temporal_impl, B=1, p_max=6, S=4, H=3, d=8, seed=2):
    """n = 1: the query sees every cached frame and itself, no mask -> SDPA."""
    g = np.random.default_rng(seed)
    ring_k = g.standard_normal((B, p_max, S, H, d))
    ring_v = g.standard_normal((B, p_max, S, H, d))
    q, k, v = (g.standard_normal((B, 1, S, H, d)) for _ in range(3))
    slots = [4, 5, 0, 1]                     # a wrapped queue of 4 frames
    scale = 0.41
    got = temporal_impl(q, k, v, ring_k, ring_v, slots, scale)
    keys = np.concatenate([ring_k[:, slots], k], 1)
    vals = np.concatenate([ring_v[:, slots], v], 1)
    perm = (0, 2, 3, 1, 4)
    ref = sdpa64(q.transpose(perm), keys.transpose(perm), vals.transpose(perm), scale)
    return float(np.max(np.abs(got.transpose(perm) - ref)))


# ---------------------------------------------------------------------------
# spatial attention
# ---------------------------------------------------------------------------
def check_spatial_vs_sdpa(spatial_impl, B=2, n=3, S=5, H=2, d=8, p=2, seed=4):
    """Prefix mode equals SDPA over the token-axis concatenation [own frame,
    prefix frames in logical order]; self mode and P' = 0 equal SDPA over the
    own frame. Returns the max error over the three cases."""
    g = np.random.default_rng(seed)
    q, k, v = (g.standard_normal((B, n, S, H, d)) for _ in range(3))
    ks, vs = (g.standard_normal((B, p + 1, S, H, d)) for _ in range(2))
    slots = [2, 0]                       # logical order != physical order
    scale = 0.33
    worst = 0.0
    got = spatial_impl(q, k, v, ks, vs, slots, scale, "prefix")
    for f in range(n):
        kk = np.concatenate([k[:, f]] + [ks[:, s] for s in slots], 1)   # [B][Sk][H][d]
        vv = np.concatenate([v[:, f]] + [vs[:, s] for s in slots], 1)
        ref = sdpa64(q[:, f].transpose(0, 2, 1, 3), kk.transpose(0, 2, 1, 3),
                     vv.transpose(0, 2, 1, 3), scale)
        worst = max(worst, float(np.max(np.abs(got[:, f].transpose(0, 2, 1, 3) - ref))))
    for mode, sl in (("self", slots), ("prefix", [])):
        got = spatial_impl(q, k, v, ks, vs, sl, scale, mode)
        for f in range(n):
            ref = sdpa64(q[:, f].transpose(0, 2, 1, 3), k[:, f].transpose(0, 2, 1, 3),
                         v[:, f].transpose(0, 2, 1, 3), scale)
            worst = max(worst, float(np.max(np.abs(got[:, f].transpose(0, 2, 1, 3) - ref))))
    return worst


def check_spatial_zero_query(spatial_impl, B=1, n=2, S=6, H=2, d=4, p=3, seed=5):
    """Q == 0: uniform weights, output = mean of all (P'+1)*S value rows."""
    g = np.random.default_rng(seed)
    q = np.zeros((B, n, S, H, d))
    k, v = (g.standard_normal((B, n, S, H, d)) for _ in range(2))
    ks, vs = (g.standard_normal((B, p, S, H, d)) for _ in range(2))
    slots = list(range(p))
    got = spatial_impl(q, k, v, ks, vs, slots, 1.0, "prefix")
    worst = 0.0
    for f in range(n):
        mean = (v[:, f].sum(1) + vs.sum((1, 2))) / ((p + 1) * S)          # [B][H][d]
        worst = max(worst, float(np.max(np.abs(got[:, f] - mean[:, None]))))
    return worst


# ---------------------------------------------------------------------------
# bidirectional temporal attention (the recompute baseline)
# ---------------------------------------------------------------------------
def check_bidirectional_vs_sdpa(bidir_impl, B=2, T=6, S=3, H=2, d=8, seed=11):
    """Every frame attends to every frame: torch's unmasked SDPA along frames."""
    g = np.random.default_rng(seed)
    q, k, v = (g.standard_normal((B, T, S, H, d)) for _ in range(3))
    scale = 0.37
    got = bidir_impl(q, k, v, scale)
    perm = (0, 2, 3, 1, 4)
    ref = sdpa64(q.transpose(perm), k.transpose(perm), v.transpose(perm), scale)
    return float(np.max(np.abs(got.transpose(perm) - ref)))


def check_bidirectional_zero_keys(bidir_impl, B=1, T=5, S=2, H=3, d=4, seed=12):
    """K == 0: every logit equal, so every query frame returns the mean of the
    values over all T frames (one-hot frame codes make any left-out or
    doubled frame visible)."""
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, T, S, H, d))
    k = np.zeros((B, T, S, H, d))
    v = np.zeros((B, T, S, H, T))
    for t in range(T):
        v[:, t, ..., t] = 1.0
    got = bidir_impl(q, k, v, 0.5)
    return float(np.max(np.abs(got - 1.0 / T)))


def check_bidirectional_permutation(bidir_impl, B=1, T=7, S=2, H=2, d=6, seed=13):
    """Permuting the frames of q, k and v permutes the output the same way;
    permuting only the key/value frames (together) leaves it unchanged."""
    g = np.random.default_rng(seed)
    q, k, v = (g.standard_normal((B, T, S, H, d)) for _ in range(3))
    perm = g.permutation(T)
    base = bidir_impl(q, k, v, 0.3)
    a = bidir_impl(q[:, perm], k[:, perm], v[:, perm], 0.3)
    b = bidir_impl(q, k[:, perm], v[:, perm], 0.3)
    return float(max(np.max(np.abs(a - base[:, perm])), np.max(np.abs(b - base))))


def check_bidirectional_last_frame_is_causal(bidir_impl, causal_impl, B=1, T=6, S=3, H=2, d=8, seed=14):
    """The last frame sees all frames under the causal mask as well, so it
    matches the causal temporal oracle (empty queue) there; the first frame,
    which sees only itself causally, must not."""
    g = np.random.default_rng(seed)
    q, k, v = (g.standard_normal((B, T, S, H, d)) for _ in range(3))
    got = bidir_impl(q, k, v, 0.3)
    causal = causal_impl(q, k, v, np.zeros((B, 1, S, H, d)), np.zeros((B, 1, S, H, d)), [], 0.3)
    last = float(np.max(np.abs(got[:, -1] - causal[:, -1])))
    first_differs = float(np.max(np.abs(got[:, 0] - causal[:, 0]))) > 1e-3
    return last if first_differs else float("inf")


# ---------------------------------------------------------------------------
# QKV projection with the cyclic TPE row (pins for qkv_proj_tpe_ref-shaped
# implementations: impl(x, w, tpe_rows, first_frame, n_frames, tokens))
# ---------------------------------------------------------------------------
# frames 11..14 with a table of 13 rows wrap after frame 12: indices written
# out by hand, not computed
_TPE_FIRST, _TPE_N, _TPE_L, _TPE_IDX = 11, 4, 13, [11, 12, 0, 1]


def check_tpe_proj_zero_input(impl, B=2, S=3, C_in=5, C=2, seed=21):
    """x = 0: every output row is exactly its frame's table row."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((3 * C, C_in))
    rows = g.standard_normal((_TPE_L, 3 * C))
    x = np.zeros((B * _TPE_N * S, C_in))
    y = np.concatenate(impl(x, w, rows, _TPE_FIRST, _TPE_N, S), 1)
    want = np.concatenate([np.repeat(rows[_TPE_IDX], S, 0)] * B, 0)
    return float(np.max(np.abs(y - want)))


def check_tpe_proj_distributive(impl, B=2, S=3, C_in=6, C=3, seed=22):
    """Table rows built as e W^T: the result equals projecting x + e[index]
    (the embedding added to the tokens first)."""
    from oracle import qkv_proj_ref
    g = np.random.default_rng(seed)
    w = g.standard_normal((3 * C, C_in))
    e = g.standard_normal((_TPE_L, C_in))
    x = g.standard_normal((B * _TPE_N * S, C_in))
    per_row = np.concatenate([np.repeat(e[_TPE_IDX], S, 0)] * B, 0)
    want = np.concatenate(qkv_proj_ref(x + per_row, w), 1)
    got = np.concatenate(impl(x, w, e @ w.T, _TPE_FIRST, _TPE_N, S), 1)
    return float(np.max(np.abs(got - want)))


# ---------------------------------------------------------------------------
# toy block layer forms (layer norm, tanh-GELU, sinusoidal timestep
# embedding, shift/scale modulation): textbook definitions, pinned by the
# mathematics since the pages do not give the backbone
# ---------------------------------------------------------------------------
LN_EPS = 1e-6


def check_layernorm(ln, seed=31):
    """What fixes a layer norm with epsilon 1e-6 over the last axis: every
    output row has mean 0 and population variance var / (var + 1e-6) (var
    the row's population variance); a constant row maps to 0; LN(a x + b) =
    LN(x) for a > 0 up to the epsilon's effect (rows of variance ~1); the
    hand-worked row [0, 0, 0, 4] (mean 1, variance 3) gives
    [-1, -1, -1, 3] / sqrt(3 + 1e-6). Returns the worst ratio of a violation
    to its tolerance (<= 1 passes)."""
    g = np.random.default_rng(seed)
    r = []
    for var_scale in (1e-7, 1e-6, 1e-3, 1.0, 50.0):   # small variances make the epsilon visible
        x = g.standard_normal((6, 9)) * np.sqrt(var_scale) + g.standard_normal((6, 1))
        y = ln(x)
        var = x.var(-1)
        r.append(float(np.max(np.abs(y.mean(-1)))) / 1e-9)
        want = var / (var + LN_EPS)
        r.append(float(np.max(np.abs(y.var(-1) - want) / want)) / 1e-9)
    r.append(float(np.max(np.abs(ln(np.full((2, 5), 3.25))))) / 1e-12)
    x = g.standard_normal((4, 16))
    r.append(float(np.max(np.abs(ln(2.5 * x - 7.0) - ln(x)))) / 1e-5)
    row = ln(np.array([[0.0, 0.0, 0.0, 4.0]]))
    want = np.array([-1.0, -1.0, -1.0, 3.0]) / np.sqrt(3.0 + 1e-6)
    r.append(float(np.max(np.abs(row - want))) / 1e-12)
    return max(r)


GELU_ERF_BOUND = 4.8e-4   # published maximum deviation of the tanh form from x*Phi(x) is ~4.73e-4


def check_gelu_tanh(gelu):
    """Worst violation of what fixes the tanh form of GELU: gelu(0) = 0;
    gelu(x) - gelu(-x) = x (tanh is odd); |gelu(x) - x Phi(x)| <= 4.8e-4 with
    Phi from math.erf; the slope of (gelu(x) - x/2) / x^2 at 0 is
    1/sqrt(2 pi), as for x Phi(x) (fixes the constant sqrt(2/pi) inside the
    tanh). Returns the worst ratio of violation to its bound (<= 1 passes)."""
    import math
    x = np.linspace(-8.0, 8.0, 4001)
    y = gelu(x)
    exact = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    r = [abs(float(gelu(np.array([0.0]))[0])) / 1e-15,
         float(np.max(np.abs(y - gelu(-x) - x))) / 1e-12,
         float(np.max(np.abs(y - exact))) / GELU_ERF_BOUND]
    h = 1e-4
    slope = (float(gelu(np.array([h]))[0]) - h / 2) / h ** 2
    r.append(abs(slope - 1.0 / math.sqrt(2.0 * math.pi)) / 1e-6)
    return max(r)


def check_timestep_embedding(temb, half):
    """What fixes the sinusoidal embedding [sin(t w_i) for i < h, cos(t w_i)
    for i < h], w_i = 1000^(-i/h): emb(0) = [0]*h + [1]*h; sin^2 + cos^2 = 1
    per frequency at any t; w_0 = 1, so emb(t)[0] = sin t and emb(t)[h] =
    cos t; the frequencies recovered from a small t by atan2 equal
    10^(-3i/h) (h = 4: 1, 0.1778279410, 0.0316227766, 0.0056234133). Returns
    the worst ratio of a violation to its tolerance (<= 1 passes)."""
    r = [float(np.max(np.abs(temb(0.0) - np.concatenate([np.zeros(half), np.ones(half)])))) / 1e-15]
    for t in (0.7, 20.0, 900.0):
        e = temb(t)
        r.append(float(np.max(np.abs(e[:half] ** 2 + e[half:] ** 2 - 1.0))) / 1e-12)
        r.append(max(abs(float(e[0]) - np.sin(t)), abs(float(e[half]) - np.cos(t))) / 1e-12)
    t = 1e-3
    e = temb(t)
    w = np.arctan2(e[:half], e[half:]) / t
    want = np.array([1.0, 0.1778279410, 0.0316227766, 0.0056234133]) if half == 4 else \
        10.0 ** (-3.0 * np.arange(half) / half)
    r.append(float(np.max(np.abs(w - want))) / 1e-9)
    return max(r)


def check_toy_modulation(model_factory, gelu, ln, S=3, C=4, seed=33):
    """The six modulation vectors of a frame (temb(t) @ wmod, split in six)
    are, in order, shift and scale of the spatial, the temporal and the MLP
    pre-norm: h = LN(x) (1 + scale) + shift. Pinned on a one-layer block with
    hand-set weights whose output has a closed form: with Q = K = 0 an
    attention layer averages its visible values (spatial: the frame's own
    tokens; temporal: frames 0..f), with the value projection and the output
    projection the identity its output is that average of the pre-norm h,
    and with w1 = [I 0], w2 = [I; 0] the MLP adds gelu(h). One layer at a
    time carries an identity value path (the others are zero), and one of the
    six vectors at a time is set to `a` through the cos(0 * w_0) = 1 entry of
    temb(0). Returns the max error against the closed forms."""
    g = np.random.default_rng(seed)
    F = 2
    x = g.standard_normal((F, S, C))
    a = g.standard_normal(C) * 0.5
    I = np.eye(C)
    worst = 0.0
    for which in range(6):
        for path in ("spatial", "temporal", "mlp"):
            m = model_factory(S=S, H=1, d=C, depth=1, temb_dim=4)
            L = m.layers[0]
            for k in L:
                L[k] = np.zeros_like(L[k])
            if path == "spatial":
                L["wqkv_s"][:, 2 * C:] = I
                L["wo_s"] = I.copy()
            elif path == "temporal":
                L["wqkv_t"][:, 2 * C:] = I
                L["wo_t"] = I.copy()
            else:
                L["w1"][:, :C] = I
                L["w2"][:C, :] = I
            L["wmod"][2, which * C:(which + 1) * C] = a      # temb(0) = [0, 0, 1, 1]
            got, _, _ = m._layer(L, x, [0] * F, [], ([], []), spatial_self=True)
            mods = [np.zeros(C)] * 6
            mods[which] = a
            lo = {"spatial": 0, "temporal": 2, "mlp": 4}[path]
            h = ln(x) * (1 + mods[lo + 1]) + mods[lo]
            if path == "spatial":
                want = x + h.mean(axis=1, keepdims=True)
            elif path == "temporal":
                want = x + np.cumsum(h, axis=0) / np.arange(1, F + 1)[:, None, None]
            else:
                want = x + gelu(h)
            worst = max(worst, float(np.max(np.abs(got - want))))
    return worst
