"""GPU parity of the cache-less entry points that serve the recompute
baseline: temporal attention over T frames (bidirectional, and causal without
a queue) and spatial self attention of T frames, through the C ABI, against
the oracle. Also: the cached path equals causal recompute over the
concatenated frames. Bars as for the cached kernels (fp32 1e-5 relative,
bf16 2e-2 max-abs)."""
import numpy as np
import pytest
import torch

import synth
from oracle import bidirectional_temporal_ref, temporal_attn_ref, spatial_attn_ref, RolloutOracle
from gpu_util import to_dev, to_host, empty_like_dev, check_close

pytestmark = pytest.mark.gpu


def frames_inputs(seed, B, T, S, H, d, dtype):
    shape = (B, T, S, H, d)
    return tuple(synth.normal(seed, x, (5, B, T, S, H, d), shape, dtype) for x in ("q", "k", "v"))


def causal_ref(q, k, v, scale):
    """Causal attention over the T frames with no queue."""
    B, T, S, H, d = q.shape
    empty = np.zeros((B, 1, S, H, d))
    return temporal_attn_ref(q, k, v, empty, empty, [], scale)


FRAME_CASES = [
    # (name, B, T, S, H, d, dtype)
    ("f32_d16_T1", 1, 1, 16, 2, 16, "f32"),
    ("f32_d16_T5", 1, 5, 16, 2, 16, "f32"),
    ("f32_d72_T17_ragged", 2, 17, 5, 3, 72, "f32"),
    ("f32_d64_T33", 1, 33, 7, 2, 64, "f32"),
    ("f32_d128_T9", 1, 9, 6, 2, 128, "f32"),
    ("bf16_d72_T1", 1, 1, 9, 3, 72, "bf16"),
    ("bf16_d72_T7", 2, 7, 5, 3, 72, "bf16"),
    ("bf16_d72_T16", 1, 16, 7, 5, 72, "bf16"),
    ("bf16_d72_T49_ragged", 1, 49, 9, 4, 72, "bf16"),
    ("bf16_d64_T20", 1, 20, 33, 2, 64, "bf16"),
    ("bf16_d128_T40", 1, 40, 6, 2, 128, "bf16"),
]
IDS = [c[0] for c in FRAME_CASES]


@pytest.mark.parametrize("name,B,T,S,H,d,dtype", FRAME_CASES, ids=IDS)
def test_bidirectional_temporal_parity(ca2, name, B, T, S, H, d, dtype):
    q, k, v = frames_inputs(31, B, T, S, H, d, dtype)
    out = empty_like_dev(q.shape, dtype)
    ca2.ca2_temporal_attn_frames(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out, causal=False)
    torch.cuda.synchronize()
    check_close(to_host(out), bidirectional_temporal_ref(q, k, v, d ** -0.5), dtype, name)


MFMA_ROW_CASES = [c for c in FRAME_CASES if c[6] == "bf16" and c[5] in (64, 72)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("name,B,T,S,H,d,dtype", MFMA_ROW_CASES, ids=[c[0] for c in MFMA_ROW_CASES])
def test_temporal_frames_matrix_core_rows(ca2, causal, name, B, T, S, H, d, dtype):
    """The matrix-core temporal kernel, forced, on the cache-less forms (T up
    to 16 runs it; longer T falls back to the dimension-split kernel)."""
    q, k, v = frames_inputs(33, B, T, S, H, d, dtype)
    out = empty_like_dev(q.shape, dtype)
    ca2.ca2_set_temporal_variant(2)
    try:
        ca2.ca2_temporal_attn_frames(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out, causal=causal)
    finally:
        ca2.ca2_set_temporal_variant(0)
    torch.cuda.synchronize()
    ref = causal_ref(q, k, v, d ** -0.5) if causal else bidirectional_temporal_ref(q, k, v, d ** -0.5)
    check_close(to_host(out), ref, dtype, f"{name} causal={causal} variant 2")


@pytest.mark.parametrize("name,B,T,S,H,d,dtype", FRAME_CASES, ids=IDS)
def test_causal_temporal_frames_parity(ca2, name, B, T, S, H, d, dtype):
    q, k, v = frames_inputs(32, B, T, S, H, d, dtype)
    out = empty_like_dev(q.shape, dtype)
    ca2.ca2_temporal_attn_frames(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out, causal=True)
    torch.cuda.synchronize()
    check_close(to_host(out), causal_ref(q, k, v, d ** -0.5), dtype, name)


SPATIAL_CASES = FRAME_CASES


@pytest.mark.parametrize("name,B,T,S,H,d,dtype", SPATIAL_CASES, ids=[c[0] for c in SPATIAL_CASES])
def test_spatial_frames_parity(ca2, name, B, T, S, H, d, dtype):
    q, k, v = frames_inputs(33, B, T, S, H, d, dtype)
    out = empty_like_dev(q.shape, dtype)
    ca2.ca2_spatial_attn_frames(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out)
    torch.cuda.synchronize()
    check_close(to_host(out), spatial_attn_ref(q, k, v, None, None, [], d ** -0.5, "self"), dtype, name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cached_path_equals_causal_recompute(ca2, dtype):
    """Queue of 9 frames + 4 new frames through the cache equals causal
    attention over the 13 concatenated frames (last 4 outputs)."""
    sh = dict(B=1, H=3, d=72, S=7, l=4, p_max=9, p_spatial=1, tpe_len=13, dtype=dtype)
    cache = ca2.Cache.from_shape(sh)
    o = RolloutOracle(sh, 41)
    for w in (1, 4, 4, 4):            # 13 frames written, queue holds the last 9
        frames = o.next_frames(w)
        cache.ca2_cache_write(*(to_dev(o.clean(x, frames), dtype) for x in ("kt", "vt", "ks", "vs")))
        o.write(frames)
    kept = o.queue.frame_ids()
    assert len(kept) == 9
    q_new, k_new, v_new = (o.noisy(x, 2, 3, 4) for x in ("q", "k", "v"))
    out_c = empty_like_dev(q_new.shape, dtype)
    cache.ca2_temporal_attn(to_dev(q_new, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype), out_c)
    # the same sequence as plain frames: queued clean K/V, then the new ones
    kq = np.concatenate([o.clean("kt", kept), k_new], axis=1)
    vq = np.concatenate([o.clean("vt", kept), v_new], axis=1)
    qq = np.concatenate([np.zeros_like(o.clean("kt", kept)), q_new], axis=1)
    out_f = empty_like_dev(qq.shape, dtype)
    ca2.ca2_temporal_attn_frames(to_dev(qq, dtype), to_dev(kq, dtype), to_dev(vq, dtype), out_f, causal=True)
    torch.cuda.synchronize()
    got_c, got_f = to_host(out_c), to_host(out_f)[:, 9:]
    check_close(got_c, got_f, dtype, "cached vs recompute")
    check_close(got_c, causal_ref(qq, kq, vq, 72 ** -0.5)[:, 9:], dtype, "cached vs oracle")


def test_recompute_rollout_last_step_sampled(ca2):
    """The recompute baseline at its largest 80-frame-rollout step (41 queued
    + 8 new = 49 frames, 256 tokens, 16 heads x 72, bf16), in the launch
    configuration the benchmark times; sampled rows / (frame, head) pairs
    checked against the oracle."""
    sh = synth.WORKLOADS["rollout_80f"]
    B, S, H, d = sh["B"], sh["S"], sh["H"], sh["d"]
    T = sh["p_max"] + sh["l"]
    q, k, v = frames_inputs(34, B, T, S, H, d, "bf16")
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    out_t = empty_like_dev(q.shape, "bf16")
    out_s = empty_like_dev(q.shape, "bf16")
    ca2.ca2_temporal_attn_frames(dq, dk, dv, out_t, causal=False)
    ca2.ca2_spatial_attn_frames(dq, dk, dv, out_s)
    torch.cuda.synchronize()
    got_t, got_s = to_host(out_t), to_host(out_s)
    g = np.random.default_rng(5)
    sc = d ** -0.5
    for s, h in zip(g.integers(0, S, 48), g.integers(0, H, 48)):
        sl = (slice(None), slice(None), slice(s, s + 1), slice(h, h + 1))
        ref = bidirectional_temporal_ref(q[sl], k[sl], v[sl], sc)
        check_close(got_t[sl], ref, "bf16", f"temporal row s={s} h={h}")
    for f, h in zip(g.integers(0, T, 6), g.integers(0, H, 6)):
        sl = (slice(None), slice(f, f + 1), slice(None), slice(h, h + 1))
        ref = spatial_attn_ref(q[sl], k[sl], v[sl], None, None, [], sc, "self")
        check_close(got_s[sl], ref, "bf16", f"spatial frame={f} h={h}")
