"""GPU cache write (K3) and cache-state parity: ring and spatial buffer bytes
bit-exact against the oracle after every write, queue frame ids / slot maps /
TPE indices bit-exact, and the cache untouched by any number of attention
calls (one shared cache serves every denoising step)."""
import numpy as np
import pytest
import torch

import synth
from oracle import RolloutOracle, tpe_index_ref
from gpu_util import to_dev, to_host, empty_like_dev, bits_to_f32

pytestmark = pytest.mark.gpu


def _host_vals(a, dtype):
    return bits_to_f32(a) if dtype == "bf16" else a


def _check_cache(cache, o, sh):
    ring_k, ring_v, sp_k, sp_v = cache.ca2_cache_debug_copy()
    ring_k, ring_v = _host_vals(ring_k, sh["dtype"]), _host_vals(ring_v, sh["dtype"])
    tids, sframes, sslots = cache.ca2_cache_frame_ids()
    assert tids == o.queue.frame_ids()
    assert cache.ca2_cache_slot_map() == o.queue.slot_map()
    info = cache.ca2_cache_info_get()
    assert info["p_k"] == o.queue.p_k and info["frames_written"] == o.frames_written
    for s in o.queue.slot_map():
        assert np.array_equal(ring_k[:, s], o.ring_k[:, s])
        assert np.array_equal(ring_v[:, s], o.ring_v[:, s])
    assert sframes == o.spatial.logical_frames()
    if sframes:
        sp_k, sp_v = _host_vals(sp_k, sh["dtype"]), _host_vals(sp_v, sh["dtype"])
        for f, s in zip(sframes, sslots):
            assert np.array_equal(sp_k[:, s], o.clean("ks", [f])[:, 0])
            assert np.array_equal(sp_v[:, s], o.clean("vs", [f])[:, 0])


@pytest.mark.parametrize("sh,writes", [
    (dict(B=1, H=2, d=16, S=16, l=4, p_max=9, p_spatial=1, tpe_len=13, dtype="f32"), [1, 4, 4, 4, 4, 2, 3]),
    (dict(B=2, H=3, d=72, S=5, l=8, p_max=25, p_spatial=3, tpe_len=33, dtype="bf16"), [1, 8, 8, 8, 8, 1, 2, 8]),
    (dict(B=1, H=2, d=72, S=8, l=8, p_max=3, p_spatial=2, tpe_len=11, dtype="bf16"), [1, 8, 2, 8]),   # n > P_max
    (dict(B=3, H=1, d=64, S=3, l=4, p_max=1, p_spatial=0, tpe_len=5, dtype="bf16"), [1, 4, 1]),
], ids=["tiny_f32", "bf16_ragged", "write_larger_than_queue", "queue_of_one"])
def test_write_bitexact_and_state(ca2, sh, writes):
    cache = ca2.Cache.from_shape(sh)
    o = RolloutOracle(sh, 31)
    for w in writes:
        frames = o.next_frames(w)
        assert cache.ca2_tpe_index(w) == tpe_index_ref(o.frames_written, w, sh["tpe_len"])
        kt, vt, ks, vs = (to_dev(o.clean(x, frames), sh["dtype"]) for x in ("kt", "vt", "ks", "vs"))
        cache.ca2_cache_write(kt, vt, ks, vs)
        o.write(frames)
        _check_cache(cache, o, sh)


def test_write_case_b4_full_queue(ca2):
    """Cache-write workload (B=4, P_max 41) from a full queue: the append
    evicts; bytes resident match the shared-cache formula."""
    sh = synth.WORKLOADS["write_b4"]
    cache = ca2.Cache.from_shape(sh)
    o = RolloutOracle(sh, 5)
    for w in [1] + [8] * 6:
        frames = o.next_frames(w)
        cache.ca2_cache_write(*(to_dev(o.clean(x, frames), "bf16") for x in ("kt", "vt", "ks", "vs")))
        o.write(frames)
    _check_cache(cache, o, sh)
    assert cache.ca2_cache_info_get()["bytes_resident"] == 207_618_048


def test_cache_unchanged_by_attention_calls(ca2):
    sh = synth.WORKLOADS["ar_step_s256"]
    cache = ca2.Cache.from_shape(sh)
    o = RolloutOracle(sh, 6)
    for w in (1, 8, 8, 8):
        frames = o.next_frames(w)
        cache.ca2_cache_write(*(to_dev(o.clean(x, frames), "bf16") for x in ("kt", "vt", "ks", "vs")))
        o.write(frames)
    before = cache.ca2_cache_debug_copy()
    out = empty_like_dev((1, 8, 256, 16, 72), "bf16")
    for t in range(50, 0, -1):
        q, k, v = (to_dev(o.noisy(x, 4, t, 8), "bf16") for x in ("q", "k", "v"))
        cache.ca2_spatial_attn(q, k, v, out)
        cache.ca2_temporal_attn(q, k, v, out)
    torch.cuda.synchronize()
    after = cache.ca2_cache_debug_copy()
    for a, b in zip(before, after):
        assert np.array_equal(a, b)


def test_errors_on_device(ca2):
    sh = dict(B=1, H=2, d=72, S=8, l=4, p_max=9, p_spatial=2, tpe_len=13, dtype="bf16")
    cache = ca2.Cache.from_shape(sh)
    x = torch.zeros((1, 4, 8, 2, 72), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    raw = ca2.load()
    # prefix mode needs a clean frame
    st = raw.ca2_spatial_attn(cache.handle, x.data_ptr(), x.data_ptr(), x.data_ptr(), out.data_ptr(), 4,
                              ca2.CA2_SPATIAL_PREFIX, 0.1, None)
    assert st == ca2.CA2_ERR_STATE
    # frame count out of range, bad mode, bad scale, misaligned pointer
    assert raw.ca2_temporal_attn(cache.handle, x.data_ptr(), x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                 5, 0.1, None) == ca2.CA2_ERR_INVALID_ARG
    assert raw.ca2_temporal_attn(cache.handle, x.data_ptr(), x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                 0, 0.1, None) == ca2.CA2_ERR_INVALID_ARG
    assert raw.ca2_spatial_attn(cache.handle, x.data_ptr(), x.data_ptr(), x.data_ptr(), out.data_ptr(), 4,
                                9, 0.1, None) == ca2.CA2_ERR_INVALID_ARG
    assert raw.ca2_temporal_attn(cache.handle, x.data_ptr(), x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                 4, float("nan"), None) == ca2.CA2_ERR_INVALID_ARG
    assert raw.ca2_temporal_attn(cache.handle, x.data_ptr() + 2, x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                 4, 0.1, None) == ca2.CA2_ERR_INVALID_ARG
    assert raw.ca2_cache_write(cache.handle, x.data_ptr(), x.data_ptr(), None, None, 4, None) == ca2.CA2_ERR_INVALID_ARG
    # nothing was written by the failed calls
    assert cache.ca2_cache_info_get()["frames_written"] == 0


def test_calls_on_a_side_stream_match_the_default_stream(ca2):
    """Every entry point runs on the caller's stream: the same writes and
    denoising calls issued on a side stream (default priority) and on the
    default stream give bit-identical caches and outputs."""
    sh = dict(B=1, H=4, d=72, S=64, l=8, p_max=9, p_spatial=3, tpe_len=17, dtype="bf16")
    outs, dumps = [], []
    side = torch.cuda.Stream()
    for stream in (None, side):
        cache = ca2.Cache.from_shape(sh)
        o = RolloutOracle(sh, 21)
        ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
        with ctx:
            for w in (1, 8, 8):
                fr = o.next_frames(w)
                cache.ca2_cache_write(*(to_dev(o.clean(x, fr), "bf16") for x in ("kt", "vt", "ks", "vs")))
                o.write(fr)
            q, k, v = (to_dev(o.noisy(x, 2, 7, 8), "bf16") for x in ("q", "k", "v"))
            ot, os_ = torch.empty_like(q), torch.empty_like(q)
            cache.ca2_spatial_attn(q, k, v, os_)
            cache.ca2_temporal_attn(q, k, v, ot)
        torch.cuda.synchronize()
        outs.append((ot.view(torch.int16).cpu(), os_.view(torch.int16).cpu()))
        dumps.append(cache.ca2_cache_debug_copy())
        cache.close()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    for a, b in zip(dumps[0], dumps[1]):
        assert np.array_equal(a, b)


def test_generation_counts_state_changes(ca2):
    """The state generation moves with every write, staging and commit, and
    with nothing else (attention calls and refused calls leave it alone), so a
    caller can tell that a captured graph's baked-in queue state is stale."""
    sh = dict(B=1, H=2, d=64, S=8, l=4, p_max=5, p_spatial=2, tpe_len=9, dtype="bf16")   # H*d multiple of 64
    B, H, d, S, l = sh["B"], sh["H"], sh["d"], sh["S"], sh["l"]
    cache = ca2.Cache.from_shape(sh, staged=True)
    x = torch.zeros((B, l, S, H, d), dtype=torch.bfloat16, device="cuda")
    gen = [cache.ca2_cache_info_get()["generation"]]
    cache.ca2_cache_write(x, x, x, x)
    gen.append(cache.ca2_cache_info_get()["generation"])
    cache.ca2_temporal_attn(x, x, x, torch.empty_like(x))
    cache.ca2_spatial_attn(x, x, x, torch.empty_like(x))
    gen.append(cache.ca2_cache_info_get()["generation"])
    xs = torch.zeros((B, l, S, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3 * H * d, 64), dtype=torch.bfloat16, device="cuda")
    cache.ca2_qkv_proj_stage(xs, w)
    gen.append(cache.ca2_cache_info_get()["generation"])
    with pytest.raises(ca2.Ca2Error):
        cache.ca2_cache_write(x, x, x, x)                    # refused while staged
    gen.append(cache.ca2_cache_info_get()["generation"])
    cache.ca2_cache_commit()
    gen.append(cache.ca2_cache_info_get()["generation"])
    torch.cuda.synchronize()
    assert gen == [0, 1, 1, 2, 2, 3]
    cache.close()
