"""Pin of the spatial prefix while fewer than P' clean frames exist (CPU).

The pages are silent on this case; the reading taken repeats the oldest held
frame in the missing logical positions, keeping (P'+1)*S keys (Ca2-VDM
notes, key design 3: the map is S x (P'+1)S; key design 5: the spatial
buffer holds the last P' frames). For that reading the oracle is pinned here
by a closed form built another way: attention over keys that repeat a frame
m times equals attention over the distinct frames in which each of that
frame's exponentials counts m times, since the repeated keys give equal
scores. The multiplicities are written out by hand for each buffer state, and
the weighted softmax is evaluated with plain loops, independently of
``spatial_attn_ref``. Planted padding mistakes each fail the pin.
"""
import math

import numpy as np
import pytest

from oracle import RolloutOracle, SpatialCache, spatial_attn_ref

SH = dict(B=1, H=2, d=8, S=4, l=4, p_max=9, p_spatial=3, tpe_len=13, dtype="f32")

# (frames written so far, in write calls) -> multiplicity of each held frame in
# the clamp-padded prefix of P' = 3 positions (hand-written)
STATES = [
    ([[0]], {0: 3}),
    ([[0], [1]], {0: 2, 1: 1}),
    ([[0], [1], [2]], {0: 1, 1: 1, 2: 1}),
    ([[0], [1, 2, 3, 4]], {2: 1, 3: 1, 4: 1}),
    ([[0, 1]], {0: 2, 1: 1}),
]


def _weighted_attention(q, k, v, kp, vp, mult, scale):
    """Own frame's keys (weight 1) + each distinct prefix frame's keys with
    weight mult[j]: sum_j w_j exp(z_j) v_j / sum_j w_j exp(z_j), by loops."""
    B, n, S, H, d = q.shape
    out = np.zeros((B, n, S, H, d))
    for b in range(B):
        for f in range(n):
            for s in range(S):
                for h in range(H):
                    keys, vals, wts = [], [], []
                    for t in range(S):
                        keys.append(k[b, f, t, h]); vals.append(v[b, f, t, h]); wts.append(1.0)
                    for j, m in enumerate(mult):
                        for t in range(S):
                            keys.append(kp[b, j, t, h]); vals.append(vp[b, j, t, h]); wts.append(float(m))
                    z = [scale * sum(float(q[b, f, s, h, e]) * float(kk[e]) for e in range(d)) for kk in keys]
                    zmax = max(z)
                    e_ = [w * math.exp(zz - zmax) for w, zz in zip(wts, z)]
                    den = sum(e_)
                    for e in range(d):
                        out[b, f, s, h, e] = sum(p * float(vv[e]) for p, vv in zip(e_, vals)) / den
    return out


def _check(cache_cls, writes, mult):
    o = RolloutOracle(SH, 5)
    o.spatial = cache_cls(SH["p_spatial"])
    for w in writes:
        o.write(w)
    q, k, v = (o.noisy(x, 1, 7, 2) for x in ("q", "k", "v"))
    got = o.spatial_out(q, k, v, "prefix")
    held = sorted(mult)
    kp, vp = o.clean("ks", held), o.clean("vs", held)
    ref = _weighted_attention(q, k, v, kp, vp, [mult[f] for f in held], o.scale)
    return float(np.max(np.abs(got - ref)))


@pytest.mark.parametrize("writes,mult", STATES)
def test_padded_prefix_is_multiplicity_weighted_attention(writes, mult):
    assert sum(mult.values()) == SH["p_spatial"]
    assert _check(SpatialCache, writes, mult) <= 1e-12


class _PadNewest(SpatialCache):          # repeats the newest held frame
    def logical_frames(self):
        h = self.held()
        return h + [h[-1]] * (self.p - len(h)) if h else []


class _NoPad(SpatialCache):              # only the held frames (fewer keys)
    def logical_frames(self):
        return self.held()


@pytest.mark.parametrize("mutant", [_PadNewest, _NoPad])
def test_padding_mistakes_fail_the_pin(mutant):
    worst = max(_check(mutant, w, m) for w, m in STATES)
    assert worst > 1e-3, mutant.__name__


def test_pin_sees_a_zero_padded_prefix():
    # zero K/V in the missing positions (a plausible mistake that keeps the
    # key count): the weighted form with the true multiplicities rejects it
    o = RolloutOracle(SH, 5)
    o.write([0])
    q, k, v = (o.noisy(x, 1, 7, 2) for x in ("q", "k", "v"))
    ks, vs = o.clean("ks", [0, 0, 0]), o.clean("vs", [0, 0, 0])
    ks[:, :2] = 0.0
    vs[:, :2] = 0.0
    bad = spatial_attn_ref(q, k, v, ks, vs, [0, 1, 2], o.scale, "prefix")
    ref = _weighted_attention(q, k, v, o.clean("ks", [0]), o.clean("vs", [0]), [3], o.scale)
    assert float(np.max(np.abs(bad - ref))) > 1e-3


def test_pin_sees_a_self_padded_prefix():
    # the target frame's own K/V in the missing positions (the self-repeat
    # form applied to the gap): rejected as well
    o = RolloutOracle(SH, 5)
    o.write([0])
    q, k, v = (o.noisy(x, 1, 7, 1) for x in ("q", "k", "v"))
    ks = np.concatenate([k, k, o.clean("ks", [0])], 1)
    vs = np.concatenate([v, v, o.clean("vs", [0])], 1)
    bad = spatial_attn_ref(q, k, v, ks, vs, [0, 1, 2], o.scale, "prefix")
    ref = _weighted_attention(q, k, v, o.clean("ks", [0]), o.clean("vs", [0]), [3], o.scale)
    assert float(np.max(np.abs(bad - ref))) > 1e-3
