"""A small spatial-temporal transformer on the GPU, through libca2 only.

Each layer: prefix-enhanced spatial attention (self attention for clean
frames), causal temporal attention over the layer's shared cache, and an MLP,
each pre-normalised and modulated by the frame's own timestep embedding
(shift and scale, adaLN style). The denoising stage reads every layer's cache
and never writes it; the cache-writing stage runs the clean chunk at
timestep 0 and stores its K/V (Ca2-VDM notes: overall framework, key designs
1-5; training section: per-frame timestep vector).

Random weights, fp32, batch 1. Every computation runs in libca2's kernels
(``ca2_toy_*`` around the attention entry points); this module only sequences
the calls and owns the buffers. It exists to check, on a real stack of
layers, that one cache serves every denoising step and that the cached
rollout reproduces a from-scratch forward over the whole sequence.
"""
from __future__ import annotations

from . import ca2

_WEIGHTS = ("wqkv_s", "wo_s", "wqkv_t", "wo_t", "w1", "w2", "wmod")


class ToyBlockGPU:
    """``layers``: one dict per layer with arrays ``wqkv_s`` [C][3C], ``wo_s``
    [C][C], ``wqkv_t`` [C][3C], ``wo_t`` [C][C], ``w1`` [C][2C], ``w2`` [2C][C]
    and ``wmod`` [temb_dim][6C] (x @ w convention)."""

    def __init__(self, layers, S, H, d, p_max, p_spatial, chunk, tpe_len=None):
        import torch
        self.S, self.H, self.d = S, H, d
        self.C = H * d
        self.chunk = chunk
        self.layers = []
        for L in layers:
            self.layers.append({k: torch.as_tensor(L[k], dtype=torch.float32).contiguous().cuda() for k in _WEIGHTS})
        self.temb_dim = self.layers[0]["wmod"].shape[0]
        self.caches = [ca2.Cache(1, H, d, S, chunk, p_max, p_spatial, tpe_len or p_max + chunk, "f32")
                       for _ in layers]

    def close(self):
        for c in self.caches:
            c.close()

    def _layer(self, W, cache, x, t, writing):
        import torch
        F, S, C = x.shape
        dev = x.device
        mod = torch.empty((F, 6 * C), dtype=torch.float32, device=dev)
        ca2.ca2_toy_temb_mod(torch.full((F,), float(t), dtype=torch.float32, device=dev), W["wmod"], mod)
        h = torch.empty_like(x)
        x2 = x.view(F * S, C)
        h2 = h.view(F * S, C)
        shape5 = (1, F, S, self.H, self.d)
        qkv = [torch.empty((F * S, C), dtype=torch.float32, device=dev) for _ in range(3)]
        att = torch.empty((F * S, C), dtype=torch.float32, device=dev)

        def project(w):
            for i in range(3):
                ca2.ca2_toy_linear(h2, w[:, i * C:(i + 1) * C], qkv[i])
            return [u.view(shape5) for u in qkv]

        # spatial attention (prefix-enhanced for targets, self for clean frames)
        ca2.ca2_toy_ln_mod(x, mod, 0, C, h)
        q, k, v = project(W["wqkv_s"])
        ks, vs = k.clone(), v.clone()
        mode = ca2.CA2_SPATIAL_SELF if writing else ca2.CA2_SPATIAL_PREFIX
        cache.ca2_spatial_attn(q, k, v, att.view(shape5), mode=mode)
        ca2.ca2_toy_linear(att, W["wo_s"], x2, r=x2)
        # causal temporal attention over the cache and the frames so far
        ca2.ca2_toy_ln_mod(x, mod, 2 * C, 3 * C, h)
        q, k, v = project(W["wqkv_t"])
        cache.ca2_temporal_attn(q, k, v, att.view(shape5))
        ca2.ca2_toy_linear(att, W["wo_t"], x2, r=x2)
        if writing:
            cache.ca2_cache_write(k, v, ks, vs)
        # MLP
        ca2.ca2_toy_ln_mod(x, mod, 4 * C, 5 * C, h)
        u = torch.empty((F * S, 2 * C), dtype=torch.float32, device=dev)
        ca2.ca2_toy_linear(h2, W["w1"], u, act=1)
        ca2.ca2_toy_linear(u, W["w2"], x2, r=x2)

    def denoise(self, x_noisy, t):
        """Denoising-stage forward of a target chunk [F][S][C] at timestep t;
        reads the caches only. Returns a new tensor."""
        x = x_noisy.clone()
        for W, c in zip(self.layers, self.caches):
            self._layer(W, c, x, t, writing=False)
        return x

    def write(self, x_clean):
        """Cache-writing stage: forward of the clean chunk at t = 0, storing
        each layer's K/V after that layer's attention. Returns the output."""
        x = x_clean.clone()
        for W, c in zip(self.layers, self.caches):
            self._layer(W, c, x, 0, writing=True)
        return x
