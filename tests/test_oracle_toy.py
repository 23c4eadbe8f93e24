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
