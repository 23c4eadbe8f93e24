"""Toy spatial-temporal transformer for the cache-sharing invariants (float64).

Test infrastructure only: the reference for the GPU run of the same block. Random weights, no
training. It exists to check, on a real stack of layers rather than on
synthetic K/V, the two properties the Ca2-VDM pages rest the method on:

1. Prefix K/V do not depend on later frames or on the denoising timestep t.
   Key design 1 (causal temporal attention: a frame sees only itself and
   earlier frames) plus key design 2 (cache sharing: clean prefix frames use
   tEmb(0), so their K/V do not depend on t), and the training section (the
   timestep vector holds 0 for the prefix and t for the targets).
2. The cached autoregressive rollout -- denoising stage reading the caches,
   cache-writing stage storing the clean chunk's K/V, FIFO queue capped at
   P_max, one-chunk spatial cache -- equals a from-scratch forward over the
   whole sequence with the equivalent attention masks (overall framework;
   key designs 3-5).

Block = spatial attention (prefix-enhanced for targets, self for clean frames)
-> causal temporal attention -> MLP, each pre-normalised and modulated by the
frame's own timestep embedding (adaLN style: shift and scale).

The layer forms (layer norm, tanh-GELU, sinusoidal timestep embedding,
shift/scale modulation) are textbook choices, since the pages do not specify
the backbone. Each is pinned by what its mathematics fixes (zero mean and the
epsilon-shrunk variance of layer norm, the odd-part identity and erf bound of
tanh-GELU, the values and frequencies of the embedding, the closed-form
roles of the modulation vectors), with planted mistakes that fail those
pins; the two cache properties above are pinned by the invariance and
full-recompute checks.
"""
from __future__ import annotations

import numpy as np

from .attention import softmax_rows


def _layernorm(x):
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(var + 1e-6)


def _gelu(x):
    return 0.5 * x * (1.0 + np.tanh(0.7978845608028654 * (x + 0.044715 * x ** 3)))


def _attend(q, k, v, scale):
    """q: [Lq][H][d], k, v: [Lk][H][d] -> [Lq][H][d] (all keys visible)."""
    z = scale * np.einsum("qhd,khd->hqk", q, k)
    p = softmax_rows(z)
    return np.einsum("hqk,khd->qhd", p, v)


class ToyModel:
    def __init__(self, seed=0, S=4, H=2, d=4, depth=2, p_max=5, p_spatial=1,
                 chunk=2, std=0.3, temb_dim=8):
        g = np.random.default_rng(seed)
        self.S, self.H, self.d, self.depth = S, H, d, depth
        self.C = H * d
        self.p_max, self.p_spatial, self.chunk = p_max, p_spatial, chunk
        self.temb_dim = temb_dim
        self.scale = 1.0 / np.sqrt(d)
        C = self.C
        self.layers = []
        for _ in range(depth):
            L = {}
            for name, shape in (("wqkv_s", (C, 3 * C)), ("wo_s", (C, C)),
                                ("wqkv_t", (C, 3 * C)), ("wo_t", (C, C)),
                                ("w1", (C, 2 * C)), ("w2", (2 * C, C)),
                                ("wmod", (temb_dim, 6 * C))):
                L[name] = g.normal(0.0, std, size=shape)
            self.layers.append(L)

    # -- timestep embedding ---------------------------------------------
    def temb(self, t):
        half = self.temb_dim // 2
        freqs = np.exp(-np.log(1000.0) * np.arange(half) / half)
        a = float(t) * freqs
        return np.concatenate([np.sin(a), np.cos(a)])

    def _mod(self, L, t):
        m = self.temb(t) @ L["wmod"]
        return np.split(m, 6)      # shift/scale for spatial, temporal, mlp

    # -- one layer on a set of frames, with explicit caches ----------------
    def _layer(self, L, x, ts, spatial_prefix, temporal_cache, spatial_self):
        """x: [F][S][C] frames processed together; ts: timestep per frame.

        spatial_prefix: list of (k, v) [S][H][d] prefix frames for the
        targets (ignored when spatial_self). temporal_cache: (k, v) lists of
        [S][H][d] earlier frames visible to every frame here (oldest first).
        Returns new x and the per-frame (spatial k, v), (temporal k, v)."""
        F = x.shape[0]
        mods = [self._mod(L, t) for t in ts]
        # spatial attention
        h = np.stack([_layernorm(x[f]) * (1 + mods[f][1]) + mods[f][0] for f in range(F)])
        qkv = (h @ L["wqkv_s"]).reshape(F, self.S, 3, self.H, self.d)
        qs, ks, vs = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        att = np.empty_like(qs)
        for f in range(F):
            if spatial_self or not spatial_prefix:
                kk, vv = ks[f], vs[f]
            else:
                kk = np.concatenate([ks[f]] + [p[0] for p in spatial_prefix], axis=0)
                vv = np.concatenate([vs[f]] + [p[1] for p in spatial_prefix], axis=0)
            att[f] = _attend(qs[f], kk, vv, self.scale)
        x = x + att.reshape(F, self.S, self.C) @ L["wo_s"]
        # causal temporal attention (per token, over frames)
        h = np.stack([_layernorm(x[f]) * (1 + mods[f][3]) + mods[f][2] for f in range(F)])
        qkv = (h @ L["wqkv_t"]).reshape(F, self.S, 3, self.H, self.d)
        qt, kt, vt = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        ck, cv = temporal_cache
        att = np.empty_like(qt)
        for f in range(F):
            keys = list(ck) + [kt[j] for j in range(f + 1)]
            vals = list(cv) + [vt[j] for j in range(f + 1)]
            K = np.stack(keys, axis=1)   # [S][J][H][d]
            V = np.stack(vals, axis=1)
            for s in range(self.S):
                att[f, s] = _attend(qt[f, s][None], K[s], V[s], self.scale)[0]
        x = x + att.reshape(F, self.S, self.C) @ L["wo_t"]
        # MLP
        h = np.stack([_layernorm(x[f]) * (1 + mods[f][5]) + mods[f][4] for f in range(F)])
        x = x + _gelu(h @ L["w1"]) @ L["w2"]
        return x, (ks, vs), (kt, vt)

    # -- cached autoregressive path ----------------------------------------
    def new_cache(self):
        return [dict(tk=[], tv=[], sk=[], sv=[]) for _ in range(self.depth)]

    def _spatial_prefix(self, c):
        if not c["sk"]:
            return []
        held = list(zip(c["sk"], c["sv"]))
        pad = [held[0]] * (self.p_spatial - len(held))
        return pad + held

    def denoise_cached(self, cache, x_noisy, t):
        """Denoising-stage forward of a target chunk at timestep t, reading
        (never writing) the caches."""
        x = np.array(x_noisy, dtype=np.float64)
        ts = [t] * x.shape[0]
        for L, c in zip(self.layers, cache):
            x, _, _ = self._layer(L, x, ts, self._spatial_prefix(c),
                                  (c["tk"], c["tv"]), spatial_self=False)
        return x

    def write_cached(self, cache, x_clean):
        """Cache-writing stage: forward of the clean chunk at t = 0 (spatial
        self mode, temporal over the queue + the chunk), then append its K/V
        to the queue (evicting past P_max) and overwrite the spatial cache."""
        x = np.array(x_clean, dtype=np.float64)
        ts = [0] * x.shape[0]
        for L, c in zip(self.layers, cache):
            x, (ks, vs), (kt, vt) = self._layer(L, x, ts, [], (c["tk"], c["tv"]),
                                                spatial_self=True)
            for f in range(x.shape[0]):
                c["tk"].append(kt[f]); c["tv"].append(vt[f])
                c["sk"].append(ks[f]); c["sv"].append(vs[f])
            del c["tk"][:-self.p_max]; del c["tv"][:-self.p_max]
            if self.p_spatial:
                del c["sk"][:-self.p_spatial]; del c["sv"][:-self.p_spatial]
            else:
                c["sk"].clear(); c["sv"].clear()
        return x

    # -- from-scratch forward over a whole sequence ----------------------------
    def forward_full(self, frames, ts, chunk_of, n_clean, prefix_temb_zero=True):
        """Forward over all frames at once, with masks instead of caches.

        frames: [N][S][C]; ts: timestep per frame; chunk_of: chunk index per
        frame (frame 0 alone is chunk 0); frames < n_clean are clean.
        A frame in a chunk starting at c0 sees temporal keys [max(0, c0 -
        P_max), itself]; a clean frame's spatial attention is self, a target's
        uses the last P' clean frames before its chunk.
        ``prefix_temb_zero=False`` gives clean frames the targets' timestep
        instead of 0 (the non-shareable baseline; used as a negative control).
        Returns final x and per-layer (spatial k, v, temporal k, v) of every frame.
        """
        x = np.array(frames, dtype=np.float64)
        N = x.shape[0]
        starts = {}
        for i, c in enumerate(chunk_of):
            starts.setdefault(c, i)
        if not prefix_temb_zero:
            t_tgt = max(ts)
            ts = [t_tgt] * N
        per_layer = []
        for L in self.layers:
            mods = [self._mod(L, t) for t in ts]
            h = np.stack([_layernorm(x[f]) * (1 + mods[f][1]) + mods[f][0] for f in range(N)])
            qkv = (h @ L["wqkv_s"]).reshape(N, self.S, 3, self.H, self.d)
            qs, ks, vs = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
            att = np.empty_like(qs)
            for f in range(N):
                c0 = starts[chunk_of[f]]
                if f < n_clean or c0 == 0:
                    kk, vv = ks[f], vs[f]
                else:
                    held = list(range(max(0, c0 - self.p_spatial), c0))
                    pre = [held[0]] * (self.p_spatial - len(held)) + held
                    kk = np.concatenate([ks[f]] + [ks[j] for j in pre], axis=0)
                    vv = np.concatenate([vs[f]] + [vs[j] for j in pre], axis=0)
                att[f] = _attend(qs[f], kk, vv, self.scale)
            x = x + att.reshape(N, self.S, self.C) @ L["wo_s"]
            h = np.stack([_layernorm(x[f]) * (1 + mods[f][3]) + mods[f][2] for f in range(N)])
            qkv = (h @ L["wqkv_t"]).reshape(N, self.S, 3, self.H, self.d)
            qt, kt, vt = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
            att = np.empty_like(qt)
            for f in range(N):
                c0 = starts[chunk_of[f]]
                w = max(0, c0 - self.p_max)
                M = np.full(N, -np.inf)
                M[w:f + 1] = 0.0
                for s in range(self.S):
                    for hh in range(self.H):
                        z = self.scale * (kt[:, s, hh] @ qt[f, s, hh]) + M
                        p = softmax_rows(z[None])[0]
                        att[f, s, hh] = p @ vt[:, s, hh]
            x = x + att.reshape(N, self.S, self.C) @ L["wo_t"]
            h = np.stack([_layernorm(x[f]) * (1 + mods[f][5]) + mods[f][4] for f in range(N)])
            x = x + _gelu(h @ L["w1"]) @ L["w2"]
            per_layer.append((ks, vs, kt, vt))
        return x, per_layer
