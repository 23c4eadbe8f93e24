"""Autoregressive rollouts on the GPU against the oracle rollout.

Tiny fp32 workload (3 AR steps x 2 denoising steps, plus one denoising call
after the last write), from both start states: every output checked. 80-frame
rollout (10 AR steps x (50 denoising calls + 1 cache-writing pass), P_max 41,
TPE table 49): every call runs on the GPU; queue, TPE and cache-writing-pass
outputs are checked at every AR step and the denoising outputs at sampled t.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import RolloutOracle, ar_schedule
from gpu_util import to_dev, to_host, empty_like_dev, check_close

pytestmark = pytest.mark.gpu


def _write_pass(cache, o, frames, dt, check=True):
    qc, kt, vt, ks, vs = (to_dev(o.clean(x, frames), dt) for x in ("qc", "kt", "vt", "ks", "vs"))
    ot = empty_like_dev(qc.shape, dt)
    os_ = empty_like_dev(qc.shape, dt)
    cache.ca2_temporal_attn(qc, kt, vt, ot)
    cache.ca2_spatial_attn(qc, ks, vs, os_, mode=1)
    cache.ca2_cache_write(kt, vt, ks, vs)
    if check:
        torch.cuda.synchronize()
        rt, rs = o.write_pass_outputs(frames)
        check_close(to_host(ot), rt, dt, f"write pass temporal {frames[0]}")
        check_close(to_host(os_), rs, dt, f"write pass spatial {frames[0]}")
    o.write(frames)


def _rollout(ca2, sh, seed, p0, ar_steps, T, check_t, extra_denoise):
    dt = sh["dtype"]
    cache = ca2.Cache.from_shape(sh)
    o = RolloutOracle(sh, seed)
    l = sh["l"]
    for frames in ar_schedule(p0, l):
        _write_pass(cache, o, frames, dt)
    p_k_seen = []
    steps = ar_steps + (1 if extra_denoise else 0)
    for ar in range(1, steps + 1):
        frames = o.next_frames(l)
        assert cache.ca2_tpe_index(l) == o.tpe(l)
        ids, _, _ = cache.ca2_cache_frame_ids()
        assert ids == o.queue.frame_ids()
        p_k_seen.append(cache.ca2_cache_info_get()["p_k"])
        ot = empty_like_dev((sh["B"], l, sh["S"], sh["H"], sh["d"]), dt)
        os_ = empty_like_dev(ot.shape, dt)
        for t in range(T, 0, -1):
            q, k, v = (to_dev(o.noisy(x, ar, t, l), dt) for x in ("q", "k", "v"))
            cache.ca2_spatial_attn(q, k, v, os_)
            cache.ca2_temporal_attn(q, k, v, ot)
            if t in check_t:
                torch.cuda.synchronize()
                rt, rs = o.denoise_outputs(ar, t)
                check_close(to_host(ot), rt, dt, f"AR {ar} t {t} temporal")
                check_close(to_host(os_), rs, dt, f"AR {ar} t {t} spatial")
        if ar <= ar_steps:
            _write_pass(cache, o, frames, dt)
    torch.cuda.synchronize()
    return p_k_seen, cache, o


def test_tiny_rollout_start_one_frame(ca2):
    sh = synth.WORKLOADS["tiny_fp32"]
    p_k, _, _ = _rollout(ca2, sh, 21, 1, 3, 2, {1, 2}, True)
    assert p_k == [1, 5, 9, 9]


def test_tiny_rollout_start_full(ca2):
    sh = synth.WORKLOADS["tiny_fp32"]
    p_k, _, o = _rollout(ca2, sh, 22, 9, 3, 2, {1, 2}, False)
    assert p_k == [9, 9, 9]
    assert o.queue.frame_ids() == list(range(12, 21))


def test_rollout_80_frames(ca2):
    sh = synth.WORKLOADS["rollout_80f"]
    p_k, cache, o = _rollout(ca2, sh, 23, 1, 10, 50, {50, 1}, False)
    assert p_k == [1, 9, 17, 25, 33, 41, 41, 41, 41, 41]
    assert o.frames_written == 81
    assert cache.ca2_cache_frame_ids()[0] == list(range(40, 81))
    assert cache.ca2_tpe_index(8) == [32, 33, 34, 35, 36, 37, 38, 39]
