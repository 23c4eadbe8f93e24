"""Toy spatial-temporal transformer: prefix K/V invariance and cached rollout
== full recompute (oracle-side, CPU)."""
import numpy as np

from oracle.toy_model import ToyModel


def _frames(n, S=4, C=8, seed=0):
    return np.random.default_rng(seed).standard_normal((n, S, C))


def test_prefix_kv_invariant_to_later_frames_and_t():
    m = ToyModel(seed=1)
    P = 5
    clean = _frames(P, seed=2)
    # chunk structure: frame 0 alone, then chunks of 2
    chunk_of = [0, 1, 1, 2, 2]
    base_x, base_kv = m.forward_full(clean, [0] * P, chunk_of, n_clean=P)
    for t, extra in ((10, 2), (700, 2), (10, 4)):
        tgt = _frames(extra, seed=3 + extra)
        co = chunk_of + [3] * 2 + ([4] * 2 if extra == 4 else [])
        _, kv = m.forward_full(np.concatenate([clean, tgt]), [0] * P + [t] * extra, co, n_clean=P)
        for (a, b) in zip(base_kv, kv):
            for x, y in zip(a, b):
                assert np.max(np.abs(x[:P] - y[:P])) <= 1e-12


def test_prefix_kv_depends_on_t_without_separate_timestep():
    # negative control: if clean frames took the targets' timestep embedding,
    # their K/V would change with t and one cache could not serve all steps
    m = ToyModel(seed=1)
    P = 5
    x = np.concatenate([_frames(P, seed=2), _frames(2, seed=9)])
    co = [0, 1, 1, 2, 2, 3, 3]
    _, kv10 = m.forward_full(x, [0] * P + [10] * 2, co, P, prefix_temb_zero=False)
    _, kv700 = m.forward_full(x, [0] * P + [700] * 2, co, P, prefix_temb_zero=False)
    diff = max(float(np.max(np.abs(a[:P] - b[:P]))) for la, lb in zip(kv10, kv700) for a, b in zip(la, lb))
    assert diff > 1e-3


def test_cached_rollout_equals_full_recompute():
    m = ToyModel(seed=4, p_max=5, p_spatial=1, chunk=2)
    l = m.chunk
    cache = m.new_cache()
    clean = _frames(1 + 5 * l, seed=5)
    m.write_cached(cache, clean[:1])
    n0 = 1
    chunk_of = [0]
    for ar in range(1, 6):
        noisy = _frames(l, seed=100 + ar)
        for t in (900, 20):
            got = m.denoise_cached(cache, noisy, t)
            seq = np.concatenate([clean[:n0], noisy])
            ref, _ = m.forward_full(seq, [0] * n0 + [t] * l, chunk_of + [ar] * l, n_clean=n0)
            assert np.max(np.abs(got - ref[n0:])) <= 1e-10, (ar, t)
        m.write_cached(cache, clean[n0:n0 + l])
        chunk_of += [ar] * l
        n0 += l
        assert len(cache[0]["tk"]) == min(n0, m.p_max)


# ---------------------------------------------------------------------------
# the block's layer forms, pinned by the mathematics (the pages do not give the
# backbone, so these are the textbook forms; the GPU toy kernels are checked
# against exactly these functions)
# ---------------------------------------------------------------------------
import math

import pytest

import pins
from oracle import toy_model


def _factory(cls=ToyModel):
    return lambda **kw: cls(seed=0, **kw)


def test_layernorm_pins():
    assert pins.check_layernorm(toy_model._layernorm) <= 1.0


def test_gelu_pins():
    assert pins.check_gelu_tanh(toy_model._gelu) <= 1.0


@pytest.mark.parametrize("temb_dim", [4, 8, 16])
def test_timestep_embedding_pins(temb_dim):
    m = ToyModel(seed=0, temb_dim=temb_dim)
    assert pins.check_timestep_embedding(m.temb, temb_dim // 2) <= 1.0


def test_modulation_order_pins():
    assert pins.check_toy_modulation(_factory(), toy_model._gelu, toy_model._layernorm) <= 1e-12


def test_zero_modulation_weights_give_plain_layernorm():
    # temb(t) @ 0 = 0 for every t: each pre-norm is LN(x) * 1 + 0
    m = ToyModel(seed=3, temb_dim=8)
    L = m.layers[0]
    L["wmod"][:] = 0.0
    for t in (0, 20, 900):
        for v in m._mod(L, t):
            assert np.all(v == 0.0)


# planted mistakes in copies of the layer forms: each must fail a pin
def _ln_no_eps(x):
    mu = x.mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(-1, keepdims=True))


def _ln_sample_var(x):
    mu = x.mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + 1e-6)


def _ln_no_center(x):
    return x / np.sqrt(x.var(-1, keepdims=True) + 1e-6)


@pytest.mark.parametrize("mutant", [_ln_no_eps, _ln_sample_var, _ln_no_center],
                         ids=["no_eps", "sample_var", "no_center"])
def test_layernorm_mutants_fail(mutant):
    with np.errstate(divide="ignore", invalid="ignore"):
        r = pins.check_layernorm(mutant)
    assert not (r <= 1.0)


def _gelu_c(c, a):
    return lambda x: 0.5 * x * (1.0 + np.tanh(c * (x + a * x ** 3)))


@pytest.mark.parametrize("mutant", [
    _gelu_c(math.sqrt(math.pi / 2), 0.044715),     # constant inverted
    _gelu_c(0.7978845608028654, 0.0),              # cubic term dropped
    _gelu_c(0.7978845608028654, 0.04),             # wrong cubic coefficient
    _gelu_c(0.8, 0.044715),                        # rounded sqrt(2/pi)
    lambda x: 0.5 * x * (1.0 - np.tanh(0.7978845608028654 * (x + 0.044715 * x ** 3))),   # sign
], ids=["inv_const", "no_cubic", "cubic_coef", "rounded_c", "sign"])
def test_gelu_mutants_fail(mutant):
    assert pins.check_gelu_tanh(mutant) > 1.0


def _temb_mutant(kind, half):
    def f(t):
        i = np.arange(half)
        if kind == "base":
            w = np.exp(-np.log(10000.0) * i / half)
        elif kind == "index":
            w = np.exp(-np.log(1000.0) * (i + 1) / half)
        else:
            w = np.exp(-np.log(1000.0) * i / half)
        a = float(t) * w
        if kind == "order":
            return np.concatenate([np.cos(a), np.sin(a)])
        return np.concatenate([np.sin(a), np.cos(a)])
    return f


@pytest.mark.parametrize("kind", ["base", "index", "order"])
def test_timestep_embedding_mutants_fail(kind):
    assert pins.check_timestep_embedding(_temb_mutant(kind, 4), 4) > 1.0


class _SwappedShiftScale(ToyModel):
    def _mod(self, L, t):
        m = super()._mod(L, t)
        return [m[1], m[0], m[3], m[2], m[5], m[4]]


class _LayerOrderSwapped(ToyModel):
    def _mod(self, L, t):
        m = super()._mod(L, t)
        return [m[2], m[3], m[0], m[1], m[4], m[5]]


@pytest.mark.parametrize("cls", [_SwappedShiftScale, _LayerOrderSwapped], ids=["shift_scale", "layer_order"])
def test_modulation_mutants_fail(cls):
    assert pins.check_toy_modulation(_factory(cls), toy_model._gelu, toy_model._layernorm) > 1e-6
