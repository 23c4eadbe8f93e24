"""The fused denoising call (ca2_denoise_attn): prefix spatial attention and
causal temporal attention of one call in one launch, on independent tensors,
against the oracle -- at the 256-token Ca2-VDM shape in the launch
configuration the benchmark step uses, on small shapes that exercise several
row blocks per workgroup, partial chunks, a growing queue, a wrapped ring,
staged frames, self mode and no spatial prefix, and on shapes that fall back
to two launches. The fused spatial half runs the same arithmetic as the
stand-alone kernel's 4 x 32-query variant and must match it bit for bit."""
import numpy as np
import pytest
import torch

from oracle import RolloutOracle, temporal_attn_ref
from gpu_util import to_dev, to_host, empty_like_dev, check_close

pytestmark = pytest.mark.gpu


def shape_of(B, H, d, S, l, p_max, p_spatial, tpe_len=None):
    return dict(B=B, H=H, d=d, S=S, l=l, p_max=p_max, p_spatial=p_spatial,
                tpe_len=tpe_len or p_max + l, dtype="bf16")


def _filled(ca2, sh, seed, writes, staged=False):
    cache = ca2.Cache.from_shape(sh, staged=staged)
    o = RolloutOracle(sh, seed)
    for w in writes:
        frames = o.next_frames(w)
        cache.ca2_cache_write(*(to_dev(o.clean(x, frames), "bf16") for x in ("kt", "vt", "ks", "vs")))
        o.write(frames)
    torch.cuda.synchronize()
    return cache, o


CASES = [
    # (name, shape, writes, n, mode, expect_fused)
    ("ar_step_s256", shape_of(1, 16, 72, 256, 8, 25, 3), [1, 8, 8, 8], 8, 0, True),
    ("s64_n1_blocks4", shape_of(1, 2, 72, 64, 8, 9, 3), [1, 8], 1, 0, True),         # 4 row blocks per workgroup
    ("s128_n3_growing", shape_of(2, 3, 72, 128, 8, 25, 3), [1, 8], 3, 0, True),      # queue not full, partial chunk
    ("s192_wrapped", shape_of(1, 2, 72, 192, 8, 9, 2), [1, 8, 8, 8, 8], 8, 0, True),  # ring wrapped, head != 0
    ("d64", shape_of(1, 4, 64, 128, 8, 25, 3), [1, 8, 8], 8, 0, True),
    ("self_mode", shape_of(1, 2, 72, 64, 8, 25, 3), [1, 8, 8], 8, 1, True),
    ("no_prefix", shape_of(1, 2, 72, 64, 4, 9, 0), [1, 4], 4, 0, True),
    ("empty_queue_self", shape_of(1, 2, 72, 64, 8, 25, 3), [], 8, 1, True),
    ("ragged_falls_back", shape_of(1, 2, 72, 100, 8, 25, 3), [1, 8], 8, 0, False),
    ("n16_falls_back", shape_of(1, 2, 72, 64, 16, 33, 3), [1, 16], 16, 0, False),
    ("d128_falls_back", shape_of(1, 2, 128, 64, 8, 17, 3), [1, 8], 8, 0, False),
    ("many_wgs_falls_back", shape_of(3, 16, 72, 128, 8, 9, 3), [1, 8], 8, 0, False),   # 384 workgroups
]


@pytest.mark.parametrize("name,sh,writes,n,mode,expect_fused", CASES, ids=[c[0] for c in CASES])
def test_denoise_call_matches_oracle(ca2, name, sh, writes, n, mode, expect_fused):
    cache, o = _filled(ca2, sh, 900, writes)
    qs, ks, vs = (o.noisy(x, 3, 1, n) for x in ("q", "k", "v"))
    qt, kt, vt = (o.noisy(x, 3, 2, n) for x in ("q", "k", "v"))     # a different work item
    dev = [to_dev(x, "bf16") for x in (qs, ks, vs, qt, kt, vt)]
    out_s = empty_like_dev(qs.shape, "bf16")
    out_t = empty_like_dev(qs.shape, "bf16")
    fused = cache.ca2_denoise_attn(*dev[:3], out_s, *dev[3:], out_t, mode=mode)
    torch.cuda.synchronize()
    assert fused == expect_fused
    ref_s = o.spatial_out(qs, ks, vs, "prefix" if mode == 0 else "self")
    check_close(to_host(out_s), ref_s, "bf16", f"{name} spatial")
    ref_t = temporal_attn_ref(qt, kt, vt, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out_t), ref_t, "bf16", f"{name} temporal")
    if fused:
        # the spatial half is the 4 x 32-query variant's arithmetic, bit for bit
        solo = empty_like_dev(qs.shape, "bf16")
        ca2.ca2_set_spatial_variant(1)
        try:
            cache.ca2_spatial_attn(*dev[:3], solo, mode=mode)
        finally:
            ca2.ca2_set_spatial_variant(0)
        torch.cuda.synchronize()
        assert torch.equal(solo, out_s), f"{name}: fused spatial half differs from the stand-alone kernel"
    cache.close()


FUSED = [c for c in CASES if c[5]]


@pytest.mark.parametrize("name,sh,writes,n,mode,expect_fused", FUSED, ids=[c[0] for c in FUSED])
def test_denoise_call_with_matrix_core_temporal(ca2, name, sh, writes, n, mode, expect_fused):
    """The fused launch with the matrix-core temporal rows forced in its
    temporal wavefronts, against the oracle; the spatial half is unchanged."""
    cache, o = _filled(ca2, sh, 903, writes)
    qs, ks, vs = (o.noisy(x, 5, 1, n) for x in ("q", "k", "v"))
    qt, kt, vt = (o.noisy(x, 5, 2, n) for x in ("q", "k", "v"))
    dev = [to_dev(x, "bf16") for x in (qs, ks, vs, qt, kt, vt)]
    out_s = empty_like_dev(qs.shape, "bf16")
    out_t = empty_like_dev(qs.shape, "bf16")
    ca2.ca2_set_temporal_variant(2)
    try:
        fused = cache.ca2_denoise_attn(*dev[:3], out_s, *dev[3:], out_t, mode=mode)
    finally:
        ca2.ca2_set_temporal_variant(0)
    torch.cuda.synchronize()
    assert fused
    check_close(to_host(out_s), o.spatial_out(qs, ks, vs, "prefix" if mode == 0 else "self"), "bf16",
                f"{name} spatial")
    ref_t = temporal_attn_ref(qt, kt, vt, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out_t), ref_t, "bf16", f"{name} temporal (matrix-core rows, fused)")
    cache.close()


def _random_fusable(n_cfg, seed):
    """Seeded shapes inside the fused launch's domain (bf16, head_dim 64 or
    72, whole 64-token tiles, n <= 8, the spatial grid within one round of 256
    workgroups), with any chunk, queue length before and after eviction, a
    wrapped ring, prefix size 0..l-1 and either spatial mode; the oracle's
    spatial work is capped so the set runs in seconds."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n_cfg:
        d = int(g.choice([64, 72]))
        S = 64 * int(g.integers(1, 5))
        B, H = int(g.integers(1, 3)), int(g.integers(1, 9))
        l = int(g.integers(1, 17))
        n = int(g.integers(1, min(l, 8) + 1))
        p_max = int(g.integers(1, 50))
        p_spatial = int(g.integers(0, min(l, 16)))
        mode = int(g.integers(0, 2))
        writes = [1] + [int(g.integers(1, l + 1)) for _ in range(int(g.integers(0, 2 * p_max // l + 3)))]
        nwg = -(-S // 128) * n * H * B
        if nwg > 256 or B * n * H * S * S * (p_spatial + 1) * d > 1.5e9:
            continue
        sh = shape_of(B, H, d, S, l, p_max, p_spatial, p_max + l + int(g.integers(0, 6)))
        out.append((f"rand{len(out)}_d{d}_B{B}H{H}S{S}_l{l}P{p_max}p{p_spatial}_w{sum(writes)}_n{n}_m{mode}",
                    sh, writes, n, mode))
    return out


RANDOM_FUSED = _random_fusable(24, 4242)


@pytest.mark.parametrize("name,sh,writes,n,mode", RANDOM_FUSED, ids=[c[0] for c in RANDOM_FUSED])
def test_denoise_call_random_shapes(ca2, name, sh, writes, n, mode):
    """Seeded shapes through the fused launch, both temporal forms, against
    the oracle; the spatial half bit-identical to the stand-alone kernel."""
    cache, o = _filled(ca2, sh, 904, writes)
    qs, ks, vs = (o.noisy(x, 6, 1, n) for x in ("q", "k", "v"))
    qt, kt, vt = (o.noisy(x, 6, 2, n) for x in ("q", "k", "v"))
    dev = [to_dev(x, "bf16") for x in (qs, ks, vs, qt, kt, vt)]
    ref_s = o.spatial_out(qs, ks, vs, "prefix" if mode == 0 and sh["p_spatial"] > 0 else "self")
    ref_t = temporal_attn_ref(qt, kt, vt, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    solo = empty_like_dev(qs.shape, "bf16")
    ca2.ca2_set_spatial_variant(1)
    try:
        cache.ca2_spatial_attn(*dev[:3], solo, mode=mode)
    finally:
        ca2.ca2_set_spatial_variant(0)
    for tv in (0, 2):
        out_s = empty_like_dev(qs.shape, "bf16")
        out_t = empty_like_dev(qs.shape, "bf16")
        ca2.ca2_set_temporal_variant(tv)
        try:
            fused = cache.ca2_denoise_attn(*dev[:3], out_s, *dev[3:], out_t, mode=mode)
        finally:
            ca2.ca2_set_temporal_variant(0)
        torch.cuda.synchronize()
        assert fused, f"{name}: expected the fused launch"
        check_close(to_host(out_s), ref_s, "bf16", f"{name} spatial (temporal variant {tv})")
        check_close(to_host(out_t), ref_t, "bf16", f"{name} temporal (variant {tv})")
        assert torch.equal(solo, out_s), f"{name}: fused spatial half differs from the stand-alone kernel"
    cache.close()


FALLBACK = [c for c in CASES if not c[5] and c[1]["d"] in (64, 72)]


@pytest.mark.parametrize("name,sh,writes,n,mode,expect_fused", FALLBACK, ids=[c[0] for c in FALLBACK])
def test_denoise_call_fallback_with_matrix_core_temporal(ca2, name, sh, writes, n, mode, expect_fused):
    """The two-launch fall-back with the matrix-core temporal kernel forced:
    the temporal half follows the forced kernel, against the oracle."""
    cache, o = _filled(ca2, sh, 901, writes)
    qs, ks, vs = (o.noisy(x, 4, 1, n) for x in ("q", "k", "v"))
    qt, kt, vt = (o.noisy(x, 4, 2, n) for x in ("q", "k", "v"))
    dev = [to_dev(x, "bf16") for x in (qs, ks, vs, qt, kt, vt)]
    out_s = empty_like_dev(qs.shape, "bf16")
    out_t = empty_like_dev(qs.shape, "bf16")
    ca2.ca2_set_temporal_variant(2)
    try:
        fused = cache.ca2_denoise_attn(*dev[:3], out_s, *dev[3:], out_t, mode=mode)
    finally:
        ca2.ca2_set_temporal_variant(0)
    torch.cuda.synchronize()
    assert not fused
    check_close(to_host(out_s), o.spatial_out(qs, ks, vs, "prefix" if mode == 0 else "self"), "bf16",
                f"{name} spatial")
    ref_t = temporal_attn_ref(qt, kt, vt, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out_t), ref_t, "bf16", f"{name} temporal (matrix-core rows)")
    cache.close()


@pytest.mark.parametrize("tv", [0, 2], ids=["dimension_split", "matrix_core_rows"])
def test_denoise_call_staged_frames(ca2, tv):
    """Write pass on a cache with staging slots: the temporal half reads the
    chunk's frames from their ring slots (k_t = v_t = NULL), the spatial half
    runs in self mode; with either temporal form in the fused launch."""
    sh = shape_of(1, 8, 72, 128, 8, 25, 3)
    cache, o = _filled(ca2, sh, 901, [1, 8, 8], staged=True)
    n, C = 8, sh["H"] * sh["d"]
    g = np.random.default_rng(5)
    # stage the clean chunk's K/V through the cache-writing projection (its
    # K/V outputs are read back: they are the new frames the temporal half
    # must find in the ring)
    import synth
    B, S, H, d = sh["B"], sh["S"], sh["H"], sh["d"]
    frames = o.next_frames(n)
    c_in = 64
    xin = synth.round_to_bf16(g.standard_normal((B, n, S, c_in)).astype(np.float32))
    w = synth.round_to_bf16((g.standard_normal((3 * C, c_in)) * 0.05).astype(np.float32))
    dx, dw = to_dev(xin, "bf16"), to_dev(w, "bf16")
    kk = empty_like_dev((B, n, S, H, d), "bf16")
    vv = empty_like_dev((B, n, S, H, d), "bf16")
    cache.ca2_qkv_proj_stage(dx, dw, None, None, kk, vv)
    torch.cuda.synchronize()
    k_new, v_new = to_host(kk).astype(np.float32), to_host(vv).astype(np.float32)   # the staged frames
    qc, kc, vc = (o.clean(x_, frames) for x_ in ("qc", "ks", "vs"))
    qt = o.noisy("q", 4, 0, n)
    dqc, dkc, dvc, dqt = (to_dev(x_, "bf16") for x_ in (qc, kc, vc, qt))
    out_s = empty_like_dev(qc.shape, "bf16")
    out_t = empty_like_dev(qc.shape, "bf16")
    ca2.ca2_set_temporal_variant(tv)
    try:
        fused = cache.ca2_denoise_attn(dqc, dkc, dvc, out_s, dqt, None, None, out_t, mode=1)
    finally:
        ca2.ca2_set_temporal_variant(0)
    torch.cuda.synchronize()
    assert fused
    check_close(to_host(out_s), o.spatial_out(qc, kc, vc, "self"), "bf16", "staged: spatial self")
    ref_t = temporal_attn_ref(qt, k_new, v_new, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)
    check_close(to_host(out_t), ref_t, "bf16", "staged: temporal")
    cache.close()


def test_denoise_call_rejects_overlap(ca2):
    sh = shape_of(1, 2, 72, 64, 8, 9, 3)
    cache, o = _filled(ca2, sh, 902, [1, 8])
    t = [empty_like_dev((1, 8, 64, 2, 72), "bf16") for _ in range(6)]
    for a in t:
        a.zero_()
    out = empty_like_dev((1, 8, 64, 2, 72), "bf16")
    with pytest.raises(ca2.Ca2Error) as e:
        cache.ca2_denoise_attn(t[0], t[1], t[2], out, t[3], t[4], t[5], out)          # one output twice
    assert e.value.status == ca2.CA2_ERR_INVALID_ARG
    with pytest.raises(ca2.Ca2Error) as e:
        cache.ca2_denoise_attn(t[0], t[1], t[2], t[3], t[3], t[4], t[5], out)         # input = other output
    assert e.value.status == ca2.CA2_ERR_INVALID_ARG
    gen = cache.ca2_cache_info_get()["generation"]
    cache.ca2_denoise_attn(t[0], t[1], t[2], out, t[0], t[1], t[2], t[4])             # shared inputs are fine
    torch.cuda.synchronize()
    assert cache.ca2_cache_info_get()["generation"] == gen
    cache.close()
