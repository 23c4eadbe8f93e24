"""The toy spatial-temporal block on the GPU (libca2 kernels only) against the
oracle's ToyModel (float64): its three helper kernels element by element, and
the cached autoregressive rollout -- one cache per layer, shared by every
denoising step -- against both the oracle's cached rollout and its
from-scratch forward over the whole sequence.

Bars. Helper kernels: the standard bound for a length-K fp32 dot product
accumulated with fused multiply-adds, |err| <= K * 2^-24 * sum_k |x_k w_k|,
plus rounding of the epilogue. End to end: |g - o| <= 1e-5 * max|o| per
output tensor: the fp32 attention bar (1e-5 relative) taken relative to the
tensor's scale, because layer normalisation and residual sums mix elements of
different sizes (measured worst case about 3e-7)."""
import numpy as np
import pytest
import torch

from oracle.toy_model import ToyModel, _layernorm, _gelu
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _toy(seed=4):
    m = ToyModel(seed=seed, S=16, H=2, d=16, depth=2, p_max=5, p_spatial=1, chunk=2, std=0.15, temb_dim=8)
    for L in m.layers:   # the weights the device holds (fp32), so both sides compute with the same values
        for k in L:
            L[k] = L[k].astype(np.float32).astype(np.float64)
    return m


def _frames(n, S=16, C=32, seed=0):
    return np.random.default_rng(seed).standard_normal((n, S, C))


@pytest.mark.parametrize("m,k,n,act,resid", [(1, 1, 1, 0, False), (37, 32, 96, 0, False), (64, 32, 64, 1, False),
                                             (50, 64, 32, 0, True), (16, 17, 33, 1, True)])
def test_toy_linear(ca2, m, k, n, act, resid):
    g = np.random.default_rng(m * 1000 + n)
    x = g.standard_normal((m, k)).astype(np.float32)
    w = (0.2 * g.standard_normal((k, n + 3))).astype(np.float32)   # a column slice of a wider matrix
    r = g.standard_normal((m, n)).astype(np.float32) if resid else None
    dx, dw = to_dev(x, "f32"), to_dev(w, "f32")
    y = to_dev(r, "f32") if resid else torch.empty((m, n), dtype=torch.float32, device="cuda")
    ca2.ca2_toy_linear(dx, dw[:, 1:n + 1], y, r=y if resid else None, act=act)   # in place when resid
    torch.cuda.synchronize()
    x64, w64 = x.astype(np.float64), w[:, 1:n + 1].astype(np.float64)
    pre = x64 @ w64
    ref = _gelu(pre) if act else pre.copy()
    if resid:
        ref += r
    # dot-product bound (GELU's slope is below 1.2), plus a few roundings of the
    # epilogue: tanh, the product, the residual add
    bound = 1.2 * k * U * (np.abs(x64) @ np.abs(w64)) + 8 * U * (np.abs(ref) + np.abs(pre))
    err = np.abs(to_host(y) - ref)
    assert np.all(err <= bound), float(np.max(err - bound))


def test_toy_ln_mod_and_temb(ca2):
    m = _toy()
    F, S, C = 3, 16, 32
    L = m.layers[0]
    t = np.array([0.0, 20.0, 900.0], dtype=np.float32)
    mod = torch.empty((F, 6 * C), dtype=torch.float32, device="cuda")
    ca2.ca2_toy_temb_mod(to_dev(t, "f32"), to_dev(L["wmod"].astype(np.float32), "f32"), mod)
    ref_mod = np.stack([m.temb(float(tt)) @ L["wmod"].astype(np.float32).astype(np.float64) for tt in t])
    got_mod = to_host(mod)
    assert np.max(np.abs(got_mod - ref_mod)) <= 1e-6 * max(1.0, np.max(np.abs(ref_mod)))
    x = _frames(F, seed=3).astype(np.float32)
    out = torch.empty((F, S, C), dtype=torch.float32, device="cuda")
    ca2.ca2_toy_ln_mod(to_dev(x, "f32"), mod, 2 * C, 3 * C, out)
    torch.cuda.synchronize()
    mods = got_mod.astype(np.float32).astype(np.float64)   # the device's own modulation values
    ref = np.stack([_layernorm(x[f].astype(np.float64)) * (1 + mods[f, 3 * C:4 * C]) + mods[f, 2 * C:3 * C]
                    for f in range(F)])
    assert np.max(np.abs(to_host(out) - ref)) <= 1e-5 * np.max(np.abs(ref))


def _close(got, ref, what):
    err = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    assert err <= 1e-5 * scale, f"{what}: max err {err:.3g} vs scale {scale:.3g}"
    return err / scale


def test_toy_rollout_cached_equals_oracle_and_recompute(ca2):
    """Conditioning frame, then 5 AR steps of chunk 2 (the queue of P_max = 5
    evicts from step 3 on); two denoising timesteps per step read the same
    caches. GPU output vs the oracle's cached rollout and vs its full-sequence
    forward with masks; cache bytes unchanged by the denoising calls."""
    from causal_kv_cache_amd.toy_block import ToyBlockGPU
    m = _toy()
    gpu = ToyBlockGPU(m.layers, m.S, m.H, m.d, m.p_max, m.p_spatial, m.chunk)
    cache = m.new_cache()
    l = m.chunk
    clean = _frames(1 + 5 * l, seed=5).astype(np.float32).astype(np.float64)
    out = gpu.write(to_dev(clean[:1], "f32"))
    ref = m.write_cached(cache, clean[:1])
    _close(to_host(out), ref, "conditioning frame write pass")
    n0, chunk_of = 1, [0]
    worst = 0.0
    for ar in range(1, 6):
        noisy = _frames(l, seed=100 + ar).astype(np.float32).astype(np.float64)
        before = [c.ca2_cache_debug_copy() for c in gpu.caches]
        for t in (900, 20):
            got = to_host(gpu.denoise(to_dev(noisy, "f32"), t))
            worst = max(worst, _close(got, m.denoise_cached(cache, noisy, t), f"ar {ar} t {t} vs cached oracle"))
            seq = np.concatenate([clean[:n0], noisy])
            full, _ = m.forward_full(seq, [0] * n0 + [t] * l, chunk_of + [ar] * l, n_clean=n0)
            worst = max(worst, _close(got, full[n0:], f"ar {ar} t {t} vs full recompute"))
        after = [c.ca2_cache_debug_copy() for c in gpu.caches]
        for b, a in zip(before, after):
            for u, w in zip(b, a):
                assert np.array_equal(u, w), "a denoising call changed the cache"
        out = gpu.write(to_dev(clean[n0:n0 + l], "f32"))
        _close(to_host(out), m.write_cached(cache, clean[n0:n0 + l]), f"ar {ar} write pass")
        chunk_of += [ar] * l
        n0 += l
        assert gpu.caches[0].ca2_cache_info_get()["p_k"] == min(n0, m.p_max)
    # the stored temporal K/V equal the oracle's cache, oldest first
    for c, oc in zip(gpu.caches, cache):
        hk, hv, _, _ = c.ca2_cache_debug_copy()
        slots = c.ca2_cache_slot_map()
        for j, s in enumerate(slots):
            _close(hk[0, s].astype(np.float64), oc["tk"][j], f"cached K frame {j}")
            _close(hv[0, s].astype(np.float64), oc["tv"][j], f"cached V frame {j}")
    gpu.close()
    print(f"toy rollout: worst max-err / max|o| = {worst:.3g}")
