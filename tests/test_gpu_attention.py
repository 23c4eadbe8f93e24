"""GPU parity of the temporal (K1) and spatial (K2) attention kernels against
the oracle, through the C ABI. fp32: |g-o| <= 1e-5|o| + 1e-6; bf16: max-abs
<= 2e-2. Shapes span several workgroup tiles and ragged tails; the full-size
workloads are checked in the launch configuration the benchmark uses."""
import numpy as np
import pytest
import torch

import synth
from oracle import RolloutOracle, temporal_attn_ref, spatial_attn_ref
from gpu_util import to_dev, to_host, empty_like_dev, check_close

pytestmark = pytest.mark.gpu


def shape_of(B, H, d, S, l, p_max, p_spatial, dtype, tpe_len=None):
    return dict(B=B, H=H, d=d, S=S, l=l, p_max=p_max, p_spatial=p_spatial,
                tpe_len=tpe_len or p_max + l, dtype=dtype)


def fill(ca2, sh, seed, writes):
    """A cache and its oracle after writing clean frames in chunks ``writes``."""
    cache = ca2.Cache.from_shape(sh)
    o = RolloutOracle(sh, seed)
    dt = sh["dtype"]
    for w in writes:
        frames = o.next_frames(w)
        kt, vt, ks, vs = (to_dev(o.clean(x, frames), dt) for x in ("kt", "vt", "ks", "vs"))
        cache.ca2_cache_write(kt, vt, ks, vs)
        o.write(frames)
    torch.cuda.synchronize()
    return cache, o


TEMPORAL_CASES = [
    # (name, shape, writes, n)
    ("tiny_f32_full_wrapped", shape_of(1, 2, 16, 16, 4, 9, 1, "f32", 13), [1, 4, 4, 4], 4),
    ("tiny_f32_full_n1", shape_of(1, 2, 16, 16, 4, 9, 1, "f32", 13), [1, 4, 4, 4], 1),
    ("tiny_f32_growing", shape_of(1, 2, 16, 16, 4, 9, 1, "f32", 13), [1, 4], 3),
    ("tiny_f32_empty", shape_of(1, 2, 16, 16, 4, 9, 1, "f32", 13), [], 4),
    ("f32_d72_ragged", shape_of(2, 3, 72, 5, 8, 25, 3, "f32"), [1, 8, 8, 8, 8], 8),
    ("f32_d32", shape_of(1, 4, 32, 9, 4, 9, 1, "f32"), [1, 4, 4, 4, 4], 4),
    ("f32_d64", shape_of(1, 3, 64, 7, 8, 9, 1, "f32"), [1, 8, 8], 5),
    ("f32_d128", shape_of(1, 2, 128, 6, 16, 17, 3, "f32"), [1, 16, 16], 16),
    ("bf16_d72_ragged", shape_of(2, 3, 72, 5, 8, 25, 3, "bf16"), [1, 8, 8, 8, 8], 8),
    ("bf16_d72_ragged_n3", shape_of(2, 3, 72, 5, 8, 25, 3, "bf16"), [1, 8, 8, 8, 8], 3),
    ("bf16_d72_n16", shape_of(1, 5, 72, 7, 16, 33, 3, "bf16"), [1, 16, 16, 16], 16),
    ("bf16_d72_empty", shape_of(1, 16, 72, 16, 8, 25, 3, "bf16"), [], 1),
    ("bf16_d64", shape_of(1, 4, 64, 33, 8, 25, 3, "bf16"), [1, 8, 8, 8, 8], 8),
    ("bf16_d128", shape_of(1, 2, 128, 40, 8, 17, 3, "bf16"), [1, 8, 8, 8], 6),
    # long queues: the ring wraps many times, head slot far from 0
    ("bf16_d72_long_ring", shape_of(1, 2, 72, 8, 8, 201, 3, "bf16", 209), [1] + [8] * 30, 8),
    ("f32_d16_long_ring", shape_of(1, 2, 16, 4, 4, 101, 1, "f32", 105), [1] + [4] * 40, 4),
    # one spatial token per frame
    ("bf16_d72_S1", shape_of(1, 3, 72, 1, 8, 25, 3, "bf16"), [1, 8, 8, 8], 8),
]


@pytest.mark.parametrize("name,sh,writes,n", TEMPORAL_CASES, ids=[c[0] for c in TEMPORAL_CASES])
def test_temporal_parity_small(ca2, name, sh, writes, n):
    cache, o = fill(ca2, sh, 100, writes)
    q, k, v = (o.noisy(x, 1, 7, n) for x in ("q", "k", "v"))
    out = empty_like_dev((sh["B"], n, sh["S"], sh["H"], sh["d"]), sh["dtype"])
    cache.ca2_temporal_attn(to_dev(q, sh["dtype"]), to_dev(k, sh["dtype"]), to_dev(v, sh["dtype"]), out)
    torch.cuda.synchronize()
    ref = temporal_attn_ref(q, k, v, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out), ref, sh["dtype"], name)


BF16_TEMPORAL = [c for c in TEMPORAL_CASES if c[1]["dtype"] == "bf16" and c[1]["d"] in (64, 72)]


@pytest.mark.parametrize("variant", [1, 2])
@pytest.mark.parametrize("name,sh,writes,n", BF16_TEMPORAL, ids=[c[0] for c in BF16_TEMPORAL])
def test_temporal_parity_each_bf16_kernel(ca2, variant, name, sh, writes, n):
    """The dimension-split VALU kernel (1) and the matrix-core rows (2), each
    forced, against the oracle."""
    cache, o = fill(ca2, sh, 100, writes)
    q, k, v = (o.noisy(x, 1, 7, n) for x in ("q", "k", "v"))
    out = empty_like_dev((sh["B"], n, sh["S"], sh["H"], sh["d"]), sh["dtype"])
    ca2.ca2_set_temporal_variant(variant)
    try:
        cache.ca2_temporal_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), out)
    finally:
        ca2.ca2_set_temporal_variant(0)
    torch.cuda.synchronize()
    ref = temporal_attn_ref(q, k, v, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out), ref, "bf16", f"{name} variant {variant}")


@pytest.mark.parametrize("variant", [1, 2])
def test_temporal_ar_step_s256_full_each_kernel(ca2, variant):
    """Both bf16 kernels at the 256-token shape, queue full, every output checked."""
    sh = synth.WORKLOADS["ar_step_s256"]
    cache, o = fill(ca2, sh, 7, [1, 8, 8, 8])
    q, k, v = (o.noisy(x, 4, 50, 8) for x in ("q", "k", "v"))
    out = empty_like_dev(q.shape, "bf16")
    ca2.ca2_set_temporal_variant(variant)
    try:
        cache.ca2_temporal_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), out)
    finally:
        ca2.ca2_set_temporal_variant(0)
    torch.cuda.synchronize()
    ref = temporal_attn_ref(q, k, v, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out), ref, "bf16", f"ar_step_s256 temporal variant {variant}")


def test_temporal_ar_step_s256_full(ca2):
    """One denoising call at the 256-token shape, queue full (P_k = 25), every output checked."""
    sh = synth.WORKLOADS["ar_step_s256"]
    cache, o = fill(ca2, sh, 7, [1, 8, 8, 8])
    assert cache.ca2_cache_info_get()["p_k"] == 25
    q, k, v = (o.noisy(x, 4, 50, 8) for x in ("q", "k", "v"))
    out = empty_like_dev(q.shape, "bf16")
    cache.ca2_temporal_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), out)
    torch.cuda.synchronize()
    ref = temporal_attn_ref(q, k, v, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out), ref, "bf16", "ar_step_s256 temporal")


def test_temporal_v_ones_is_exact_one(ca2):
    sh = shape_of(1, 16, 72, 32, 8, 25, 3, "bf16")
    cache = ca2.Cache.from_shape(sh)
    g = np.random.default_rng(0)
    for w in (1, 8, 8, 8, 8):
        kt = synth.round_to_bf16(g.standard_normal((1, w, 32, 16, 72)).astype(np.float32) * 3)
        ones = np.ones_like(kt)
        cache.ca2_cache_write(to_dev(kt, "bf16"), to_dev(ones, "bf16"), to_dev(kt, "bf16"), to_dev(ones, "bf16"))
    q = synth.round_to_bf16(g.standard_normal((1, 8, 32, 16, 72)).astype(np.float32) * 3)
    out = empty_like_dev(q.shape, "bf16")
    cache.ca2_temporal_attn(to_dev(q, "bf16"), to_dev(q, "bf16"), to_dev(np.ones_like(q), "bf16"), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), np.ones(q.shape))


def test_temporal_never_reads_unwritten_slots(ca2, monkeypatch):
    """Ring filled with NaN before any write: a partly filled queue must give finite outputs."""
    monkeypatch.setenv("CA2_NAN_CANARY", "1")
    sh = shape_of(1, 4, 72, 24, 8, 25, 3, "bf16")
    cache, o = fill(ca2, sh, 3, [1, 8])
    ring = cache.ca2_cache_debug_copy()[0]
    assert np.all(ring[:, 9:] == 0xFFFF)       # slots 9.. still hold the canary
    q, k, v = (o.noisy(x, 2, 3, 8) for x in ("q", "k", "v"))
    out = empty_like_dev(q.shape, "bf16")
    cache.ca2_temporal_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), out)
    torch.cuda.synchronize()
    ref = temporal_attn_ref(q, k, v, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out), ref, "bf16", "canary temporal")


SPATIAL_CASES = [
    # (name, shape, writes, n, mode)
    ("tiny_f32_prefix_clamp", shape_of(1, 2, 16, 16, 4, 9, 1, "f32", 13), [1], 4, 0),
    ("tiny_f32_prefix", shape_of(1, 2, 16, 16, 4, 9, 1, "f32", 13), [1, 4, 4], 4, 0),
    ("tiny_f32_self", shape_of(1, 2, 16, 16, 4, 9, 1, "f32", 13), [1, 4], 4, 1),
    ("f32_d72_ragged_prefix", shape_of(2, 3, 72, 70, 8, 25, 3, "f32"), [1, 8], 3, 0),
    ("f32_d128_self", shape_of(1, 2, 128, 65, 8, 25, 3, "f32"), [1], 2, 1),
    ("bf16_d72_ragged_prefix_clamp", shape_of(2, 3, 72, 200, 8, 25, 3, "bf16"), [1], 8, 0),
    ("bf16_d72_ragged_prefix", shape_of(2, 3, 72, 200, 8, 25, 3, "bf16"), [1, 8, 1], 8, 0),
    ("bf16_d72_ragged_self", shape_of(2, 3, 72, 200, 8, 25, 3, "bf16"), [1, 8], 5, 1),
    ("bf16_d72_p0", shape_of(1, 2, 72, 130, 4, 9, 0, "bf16"), [1, 4], 4, 0),
    ("bf16_d72_tiny_tokens", shape_of(1, 3, 72, 9, 4, 9, 2, "bf16"), [1, 4], 4, 0),
    ("bf16_d64_prefix", shape_of(1, 4, 64, 192, 8, 25, 3, "bf16"), [1, 8], 8, 0),
    ("bf16_d128_prefix", shape_of(1, 2, 128, 100, 8, 25, 2, "bf16"), [1, 8], 4, 0),
    # the largest prefix (P' = chunk - 1 = 15 frames, 16 key frames), filled and clamp-padded
    ("bf16_d72_max_prefix", shape_of(1, 2, 72, 40, 16, 17, 15, "bf16", 33), [1, 16, 16], 16, 0),
    ("bf16_d72_max_prefix_clamp", shape_of(1, 2, 72, 40, 16, 17, 15, "bf16", 33), [1], 16, 0),
    ("bf16_d128_max_prefix", shape_of(1, 1, 128, 17, 16, 17, 15, "bf16", 33), [1, 16], 3, 0),
    ("f32_d16_max_prefix", shape_of(1, 2, 16, 16, 16, 17, 15, "f32", 33), [1, 16], 5, 0),
    # one token per frame: one real key per key frame, the rest of each tile masked
    ("bf16_d64_S1", shape_of(1, 3, 64, 1, 4, 9, 2, "bf16"), [1, 4], 4, 0),
    ("bf16_d64_S1_self", shape_of(1, 3, 64, 1, 4, 9, 2, "bf16"), [1, 4], 4, 1),
]


@pytest.mark.parametrize("name,sh,writes,n,mode", SPATIAL_CASES, ids=[c[0] for c in SPATIAL_CASES])
def test_spatial_parity_small(ca2, name, sh, writes, n, mode):
    cache, o = fill(ca2, sh, 200, writes)
    q, k, v = (o.noisy(x, 1, 9, n) for x in ("q", "k", "v"))
    out = empty_like_dev(q.shape, sh["dtype"])
    cache.ca2_spatial_attn(to_dev(q, sh["dtype"]), to_dev(k, sh["dtype"]), to_dev(v, sh["dtype"]), out, mode=mode)
    torch.cuda.synchronize()
    ref = o.spatial_out(q, k, v, "prefix" if mode == 0 else "self")
    check_close(to_host(out), ref, sh["dtype"], name)


def test_spatial_ar_step_s256_full(ca2):
    sh = synth.WORKLOADS["ar_step_s256"]
    cache, o = fill(ca2, sh, 8, [1, 8, 8, 8])
    q, k, v = (o.noisy(x, 4, 50, 8) for x in ("q", "k", "v"))
    out = empty_like_dev(q.shape, "bf16")
    cache.ca2_spatial_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), out)
    torch.cuda.synchronize()
    ref = o.spatial_out(q, k, v, "prefix")
    check_close(to_host(out), ref, "bf16", "ar_step_s256 spatial")


def test_spatial_v_ones(ca2):
    sh = shape_of(1, 2, 72, 256, 8, 25, 3, "bf16")
    cache = ca2.Cache.from_shape(sh)
    g = np.random.default_rng(1)
    kt = synth.round_to_bf16(g.standard_normal((1, 8, 256, 2, 72)).astype(np.float32) * 3)
    ones = np.ones_like(kt)
    cache.ca2_cache_write(to_dev(kt, "bf16"), to_dev(ones, "bf16"), to_dev(kt, "bf16"), to_dev(ones, "bf16"))
    out = empty_like_dev(kt.shape, "bf16")
    cache.ca2_spatial_attn(to_dev(kt, "bf16"), to_dev(kt, "bf16"), to_dev(ones, "bf16"), out)
    torch.cuda.synchronize()
    # P is rounded to bf16 for the PV product while the normaliser stays fp32
    assert np.max(np.abs(to_host(out) - 1.0)) <= 2.0 ** -7


def test_large_b8_s1024_sampled(ca2):
    """Batched 32x32-latent workload at full size: both kernels in their
    benchmark launch configuration, outputs sampled over tokens (rows are
    independent, so the oracle runs on those tokens only)."""
    sh = synth.WORKLOADS["large_b8_s1024"]
    cache, o = fill(ca2, sh, 9, [1, 8, 8, 8])
    q, k, v = (o.noisy(x, 4, 50, 8) for x in ("q", "k", "v"))
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    ot = empty_like_dev(q.shape, "bf16")
    os_ = empty_like_dev(q.shape, "bf16")
    cache.ca2_temporal_attn(dq, dk, dv, ot)
    cache.ca2_spatial_attn(dq, dk, dv, os_)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    toks = np.unique(np.concatenate([[0, 1, 63, 64, 511, 1022, 1023], g.integers(0, 1024, 25)]))
    # temporal: slice tokens of every operand
    ref_t = temporal_attn_ref(q[:, :, toks], k[:, :, toks], v[:, :, toks],
                              o.ring_k[:, :, toks], o.ring_v[:, :, toks], o.queue.slot_map(), o.scale)
    check_close(to_host(ot)[:, :, toks], ref_t, "bf16", "large temporal")
    # spatial: slice query tokens only (keys stay whole); two batch entries, all frames/heads
    for b in (0, 7):
        ks, vs, slots = o.spatial_prefix()
        ref_s = spatial_attn_ref(q[b:b + 1, :, toks], k[b:b + 1], v[b:b + 1], ks[b:b + 1], vs[b:b + 1],
                                 slots, o.scale, "prefix")
        check_close(to_host(os_)[b:b + 1, :, toks], ref_s, "bf16", f"large spatial b={b}")


FULL_TILE_CASES = [
    # token counts that are whole 64-key tiles (the exact-count copy waits)
    ("bf16_d72_S64_prefix", shape_of(2, 3, 72, 64, 8, 25, 3, "bf16"), [1, 8, 8], 8, 0),
    ("bf16_d72_S256_prefix", shape_of(1, 2, 72, 256, 8, 25, 3, "bf16"), [1, 8, 8, 8], 8, 0),
    ("bf16_d72_S512_clamp", shape_of(1, 1, 72, 512, 4, 9, 3, "bf16"), [1], 3, 0),
    ("bf16_d72_S128_self", shape_of(1, 3, 72, 128, 8, 25, 3, "bf16"), [1, 8], 5, 1),
    ("bf16_d64_S192_prefix", shape_of(1, 2, 64, 192, 8, 25, 2, "bf16"), [1, 8, 8], 6, 0),
    ("bf16_d72_S1024_p1", shape_of(1, 1, 72, 1024, 4, 9, 1, "bf16"), [1, 4], 2, 0),
]


@pytest.mark.parametrize("cfg", ["1", "2", "3", "4"])
@pytest.mark.parametrize("name,sh,writes,n,mode",
                         [c for c in SPATIAL_CASES if c[1]["dtype"] == "bf16"] + FULL_TILE_CASES,
                         ids=[c[0] for c in SPATIAL_CASES if c[1]["dtype"] == "bf16"] + [c[0] for c in FULL_TILE_CASES])
def test_spatial_parity_every_launch_variant(ca2, cfg, name, sh, writes, n, mode):
    """Every bf16 launch variant (4 wavefronts x 32 queries, 4 x 64 queries,
    8 wavefronts = 4 x 32 queries x 2 key halves, 4 x 32 queries plus a
    wavefront that issues every copy) against the oracle, whatever the grid
    size would pick."""
    if cfg == "2" and sh["d"] > 72:
        pytest.skip("64-query wavefronts are built for d <= 72 only")
    cache, o = fill(ca2, sh, 300, writes)
    q, k, v = (o.noisy(x, 2, 4, n) for x in ("q", "k", "v"))
    out = empty_like_dev(q.shape, "bf16")
    ca2.ca2_set_spatial_variant(int(cfg))
    try:
        cache.ca2_spatial_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), out, mode=mode)
    finally:
        ca2.ca2_set_spatial_variant(0)
    torch.cuda.synchronize()
    ref = o.spatial_out(q, k, v, "prefix" if mode == 0 else "self")
    check_close(to_host(out), ref, "bf16", f"{name} cfg {cfg}")


def _random_configs(n_cfg, seed):
    """Seeded samples over the supported domain (both dtypes, every built
    head_dim, ragged token counts, any chunk, queue and prefix size, partial
    chunks, queues before and after eviction), with the spatial oracle's work
    capped so the whole set runs in seconds."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n_cfg:
        dtype = ["f32", "bf16"][g.integers(2)]
        d = int(g.choice([16, 32, 64, 72, 128] if dtype == "f32" else [64, 72, 128]))
        B, H, S = int(g.integers(1, 4)), int(g.integers(1, 6)), int(g.integers(1, 140))
        l = int(g.integers(1, 17))
        p_max = int(g.integers(1, 61))
        p_spatial = int(g.integers(0, l))
        writes = [1] + [int(g.integers(1, l + 1)) for _ in range(int(g.integers(0, 2 * p_max // l + 3)))]
        n = int(g.integers(1, l + 1))
        if B * n * H * S * S * (p_spatial + 1) * d > 1.5e9:
            continue
        sh = shape_of(B, H, d, S, l, p_max, p_spatial, dtype, p_max + l + int(g.integers(0, 6)))
        out.append((f"rand{len(out)}_{dtype}_d{d}_B{B}H{H}S{S}_l{l}P{p_max}p{p_spatial}_w{sum(writes)}_n{n}",
                    sh, writes, n))
    return out


RANDOM_CASES = _random_configs(40, 2024)


@pytest.mark.parametrize("name,sh,writes,n", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_random_configs_both_kernels(ca2, name, sh, writes, n):
    cache, o = fill(ca2, sh, 300, writes)
    q, k, v = (o.noisy(x, 2, 11, n) for x in ("q", "k", "v"))
    dq, dk, dv = (to_dev(x, sh["dtype"]) for x in (q, k, v))
    out_t = empty_like_dev(q.shape, sh["dtype"])
    out_s = empty_like_dev(q.shape, sh["dtype"])
    cache.ca2_temporal_attn(dq, dk, dv, out_t)
    cache.ca2_spatial_attn(dq, dk, dv, out_s, mode=0)
    torch.cuda.synchronize()
    check_close(to_host(out_t), temporal_attn_ref(q, k, v, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale),
                sh["dtype"], name + " temporal")
    check_close(to_host(out_s), o.spatial_out(q, k, v, "prefix"), sh["dtype"], name + " spatial")
    assert cache.ca2_cache_frame_ids()[0] == o.queue.frame_ids()


@pytest.mark.parametrize("kernel,log2a", [("temporal", 52), ("spatial", 11)])
@pytest.mark.parametrize("pattern", ["uniform", "tiered", "late_max"])
def test_large_negative_scores(ca2, pattern, kernel, log2a):
    """Inputs of magnitude 2^log2a (bf16-exact) with every score negative.
    Temporal at 2^52: every scaled score is about -1e32 in base 2, far below
    any finite starting sentinel short of the float range, so the running
    maximum must be taken from the scores themselves. Spatial at 2^11 (scores
    about -5e7): the largest magnitude its exp2(fma(s, c, -m)) form supports
    with margin (the fma's rounding residue is a common factor of every P,
    which cancels, as long as it cannot overflow: |scaled score| < 2^31).
    With equal keys the output is the mean of the cached values; with tiered
    keys it is the mean of the values of the least negative tier (one-hot up
    to ties at these gaps); either way the oracle's. late_max puts the new
    frames' keys above every cached tier, so the maximum jumps by ~1e7 (base
    2) when the last keys arrive: the raise must bring those keys' scores onto
    the new maximum exactly alike (the spatial kernel re-scores the chunk with
    the new maximum inside its product), and the output is the mean of the new
    frames' values."""
    from oracle import TemporalQueue, SpatialCache
    B, H, d, S, l, P, Ps = 1, 2, 72, 64, 8, 8, 3
    sh = shape_of(B, H, d, S, l, P, Ps, "bf16")
    a = 2.0 ** log2a
    g = np.random.default_rng(7)
    ones = np.ones((B, l, S, H, d), np.float32)
    tier = np.ones_like(ones)
    if pattern in ("tiered", "late_max"):
        tier *= (1.0 + (np.arange(l) % 4) / 4.0)[None, :, None, None, None]   # 1, 1.25, 1.5, 1.75
    k_clean = (-a * tier).astype(np.float32)
    v_clean = synth.round_to_bf16(g.standard_normal(ones.shape).astype(np.float32))
    cache = ca2.Cache.from_shape(sh)
    kd, vd = to_dev(k_clean, "bf16"), to_dev(v_clean, "bf16")
    cache.ca2_cache_write(kd, vd, kd, vd)
    q = (a * ones).astype(np.float32)
    # below every cached tier, or (late_max) above them all
    k_new = ((-0.5 if pattern == "late_max" else -2.0) * a * ones).astype(np.float32)
    v_new = synth.round_to_bf16(g.standard_normal(ones.shape).astype(np.float32))
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k_new, v_new))
    out = empty_like_dev(q.shape, "bf16")
    if kernel == "temporal":
        cache.ca2_temporal_attn(dq, dk, dv, out)
    else:
        cache.ca2_spatial_attn(dq, dk, dv, out)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    if kernel == "temporal":
        tq = TemporalQueue(P)
        tq.write(range(l))
        ring_k = np.zeros((B, P, S, H, d), np.float32)
        ring_v = np.zeros_like(ring_k)
        ring_k[:, :l], ring_v[:, :l] = k_clean, v_clean
        ref = temporal_attn_ref(q, k_new, v_new, ring_k, ring_v, tq.slot_map(), scale)
    else:
        sc = SpatialCache(Ps)
        sc.write(range(l))
        frames = sc.logical_frames()
        ref = spatial_attn_ref(q, k_new, v_new, k_clean[:, frames], v_clean[:, frames], list(range(Ps)),
                               scale, "prefix")
    check_close(to_host(out), ref, "bf16", f"{pattern} {kernel}")
    cache.close()
