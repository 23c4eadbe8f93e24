"""The cache-writing projection with the cache write fused into it
(ca2_cache_create_staged, ca2_qkv_proj_stage, ca2_cache_commit).

Parity: the projection's Q/K/V against the oracle's projection with the
cyclic TPE row (bf16 bar, max-abs 2e-2); the write-pass temporal attention
that reads the staged frames from the ring, and the denoising calls after the
commit, against the oracle's attention over the oracle's own K/V (its
projection rounded once to bf16); queue placement bit-exact against the
oracle queue with P_max + l physical slots; ring and spatial buffer contents
bit-identical to the K/V the same call wrote to the caller's buffers; and,
without a TPE table, the whole cache bit-identical to the unfused path
(ca2_qkv_proj, then ca2_cache_write)."""
import numpy as np
import pytest
import torch

import synth
from oracle import (qkv_proj_tpe_ref, temporal_attn_ref, spatial_attn_ref, TemporalQueue,
                    SpatialCache)
from gpu_util import to_dev, to_host, bits_to_f32, check_close

pytestmark = pytest.mark.gpu

RING, SPATIAL = 1, 2
# B2 H2 d64 (C = 128: a 256-wide and a 128-wide channel tile of the 384
# outputs), 40 tokens (chunk rows 2*4*40 = 320: two token tiles, ragged), P_max
# 5 with 9 ring slots, TPE table 9 (wraps at frame 9)
SMALL = dict(B=2, H=2, d=64, S=40, l=4, p_max=5, p_spatial=2, tpe_len=9, dtype="bf16")
C_IN = 128


def _bf16(a):
    return synth.round_to_bf16(np.asarray(a, np.float32)).astype(np.float64)


def _inputs(sh, c_in, seed, n, step):
    B, S = sh["B"], sh["S"]
    return synth.normal(seed, "x", (3, step, B, n, S, c_in), (B * n * S, c_in), "bf16")


def _weights(sh, c_in, seed, tpe_scale=0.5):
    C = sh["H"] * sh["d"]
    w = synth.weight(seed, 3 * C, c_in, 0.05)
    rows = synth.normal(seed, "w", (4, sh["tpe_len"], 3 * C), (sh["tpe_len"], 3 * C), "f32", std=tpe_scale)
    return w, rows


def _split(y, sh, n):
    """[M][C] -> [B][n][S][H][d]"""
    return np.asarray(y).reshape(sh["B"], n, sh["S"], sh["H"], sh["d"])


@pytest.mark.parametrize("temporal_variant", [0, 2])
def test_staged_rollout_against_oracle(ca2, temporal_variant):
    """Conditioning frame, then 4 chunks of 4 (17 frames): the queue evicts,
    the 9 ring slots and the 9-entry TPE table both wrap. Each chunk: stage
    (ring + spatial), the write pass's temporal attention over the staged
    frames, commit, then one denoising call on the committed cache. Run with
    the default temporal kernel and with the matrix-core rows forced (their
    new keys then come from the ring's staging slots too)."""
    ca2.ca2_set_temporal_variant(temporal_variant)
    try:
        _staged_rollout(ca2)
    finally:
        ca2.ca2_set_temporal_variant(0)


def _staged_rollout(ca2):
    sh = SMALL
    B, S, H, d, l, P, Ps = sh["B"], sh["S"], sh["H"], sh["d"], sh["l"], sh["p_max"], sh["p_spatial"]
    scale = d ** -0.5
    cache = ca2.Cache.from_shape(sh, staged=True)
    assert cache.ca2_cache_info_get()["ring_slots"] == P + l
    w, rows = _weights(sh, C_IN, 31)
    dw, drows = to_dev(w, "bf16"), torch.from_numpy(rows.astype(np.float32)).cuda()
    oq = TemporalQueue(P, slots=P + l)
    osp = SpatialCache(Ps)
    ok_frames, ov_frames = {}, {}       # oracle K/V (bf16-rounded) of every clean frame by id
    fw = 0
    for step, n in enumerate([1, l, l, l, l]):
        x = _inputs(sh, C_IN, 7, n, step)
        exact = [_split(t, sh, n) for t in qkv_proj_tpe_ref(x, w, rows, fw, n, S)]
        q_ref, k_ref, v_ref = (_bf16(t) for t in exact)   # the oracle's K/V as stored in bf16
        dq, dk, dv = (torch.empty((B, n, S, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
        cache.ca2_qkv_proj_stage(to_dev(x, "bf16").view(B, n, S, C_IN), dw, drows, dq, dk, dv)
        info = cache.ca2_cache_info_get()
        assert info["staged_frames"] == n and info["frames_written"] == fw
        # write pass: temporal attention of the chunk over the queue before eviction + the staged frames
        out = torch.empty_like(dq)
        cache.ca2_temporal_attn(dq, None, None, out)
        torch.cuda.synchronize()
        for got, ref, nm in zip((dq, dk, dv), exact, "qkv"):
            check_close(to_host(got), ref, "bf16", f"step {step} projected {nm}")
        ids = oq.frame_ids()
        rk = np.stack([ok_frames[f] for f in ids], 1) if ids else np.zeros((B, 0, S, H, d))
        rv = np.stack([ov_frames[f] for f in ids], 1) if ids else np.zeros((B, 0, S, H, d))
        ref_t = temporal_attn_ref(q_ref, k_ref, v_ref, rk, rv, list(range(len(ids))), scale)
        check_close(to_host(out), ref_t, "bf16", f"step {step} write-pass temporal attention")
        # ring and spatial buffer hold exactly the bits written to the caller's k / v
        hk, hv, hks, hvs = cache.ca2_cache_debug_copy()
        kb = dk.view(torch.int16).cpu().numpy().view(np.uint16)
        vb = dv.view(torch.int16).cpu().numpy().view(np.uint16)
        for f in range(n):
            slot = (fw + f) % (P + l)
            assert np.array_equal(hk[:, slot], kb[:, f]) and np.array_equal(hv[:, slot], vb[:, f])
            if f >= n - Ps:
                ss = (fw + f) % Ps
                assert np.array_equal(hks[:, ss], kb[:, f]) and np.array_equal(hvs[:, ss], vb[:, f])
        cache.ca2_cache_commit()
        landed = oq.write(range(fw, fw + n))
        osp.write(range(fw, fw + n))
        for f in range(n):
            ok_frames[fw + f], ov_frames[fw + f] = k_ref[:, f], v_ref[:, f]
        fw += n
        info = cache.ca2_cache_info_get()
        assert info["staged_frames"] == 0 and info["frames_written"] == fw and info["p_k"] == oq.p_k
        assert cache.ca2_cache_slot_map() == oq.slot_map()
        assert [(fw - n + f) % (P + l) for f in range(n)] == landed
        # a denoising call on the committed cache: prefix spatial + causal temporal
        qn, kn, vn = (synth.step_tensor(9, nm, step, 0, B, l, S, H, d, "bf16") for nm in ("q", "k", "v"))
        dqn, dkn, dvn = (to_dev(t, "bf16") for t in (qn, kn, vn))
        ot, os_ = torch.empty_like(dqn), torch.empty_like(dqn)
        cache.ca2_temporal_attn(dqn, dkn, dvn, ot)
        cache.ca2_spatial_attn(dqn, dkn, dvn, os_)
        torch.cuda.synchronize()
        ids = oq.frame_ids()
        rk = np.stack([ok_frames[f] for f in ids], 1)
        rv = np.stack([ov_frames[f] for f in ids], 1)
        check_close(to_host(ot), temporal_attn_ref(qn, kn, vn, rk, rv, list(range(len(ids))), scale), "bf16",
                    f"step {step} denoising temporal")
        pf = osp.logical_frames()
        ks = np.stack([ok_frames[f] for f in pf], 1)
        vs = np.stack([ov_frames[f] for f in pf], 1)
        check_close(to_host(os_), spatial_attn_ref(qn, kn, vn, ks, vs, list(range(Ps)), scale, "prefix"), "bf16",
                    f"step {step} denoising spatial prefix")
    cache.close()


def test_staged_without_tpe_equals_unfused_path_bitwise(ca2):
    """No TPE table: the fused stage + commit leaves the cache bit-identical to
    the plain projection followed by ca2_cache_write (same ring placement),
    over writes that evict; Q/K/V outputs identical too."""
    sh = SMALL
    B, S, H, d, l = sh["B"], sh["S"], sh["H"], sh["d"], sh["l"]
    C = H * d
    fused = ca2.Cache.from_shape(sh, staged=True)
    plain = ca2.Cache.from_shape(sh, staged=True)
    w, _ = _weights(sh, C_IN, 32)
    dw = to_dev(w, "bf16")
    for step, n in enumerate([1, l, l, 3, l]):
        dx = to_dev(_inputs(sh, C_IN, 8, n, step), "bf16")
        q1, k1, v1, q2, k2, v2 = (torch.empty((B, n, S, H, d), dtype=torch.bfloat16, device="cuda")
                                  for _ in range(6))
        fused.ca2_qkv_proj_stage(dx.view(B, n, S, C_IN), dw, None, q1, k1, v1)
        fused.ca2_cache_commit()
        ca2.ca2_qkv_proj(dx, dw, q2.view(-1, C), k2.view(-1, C), v2.view(-1, C))
        plain.ca2_cache_write(k2, v2, k2, v2)
        torch.cuda.synchronize()
        for a, b in ((q1, q2), (k1, k2), (v1, v2)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        for a, b in zip(fused.ca2_cache_debug_copy(), plain.ca2_cache_debug_copy()):
            assert np.array_equal(a, b), f"step {step}"
        assert fused.ca2_cache_slot_map() == plain.ca2_cache_slot_map()
    fused.close()
    plain.close()


def test_two_layer_projections_ring_then_spatial(ca2):
    """The temporal layer's projection (with TPE) fills the ring and the
    spatial layer's (another weight, no TPE) the spatial buffer, as two calls
    for the same chunk; caller outputs left NULL. The commit needs both."""
    sh = SMALL
    B, S, H, d, l, P, Ps = sh["B"], sh["S"], sh["H"], sh["d"], sh["l"], sh["p_max"], sh["p_spatial"]
    cache = ca2.Cache.from_shape(sh, staged=True)
    wt, rows = _weights(sh, C_IN, 33)
    ws, _ = _weights(sh, C_IN, 34)
    dwt, dws = to_dev(wt, "bf16"), to_dev(ws, "bf16")
    drows = torch.from_numpy(rows.astype(np.float32)).cuda()
    fw = 0
    for step, n in enumerate([1, l, l]):
        x = _inputs(sh, C_IN, 10, n, step)
        dx = to_dev(x, "bf16").view(B, n, S, C_IN)
        cache.ca2_qkv_proj_stage(dx, dwt, drows, targets=RING)
        with pytest.raises(ca2.Ca2Error) as e:
            cache.ca2_cache_commit()              # spatial buffer not staged yet
        assert e.value.status == ca2.CA2_ERR_STATE
        cache.ca2_qkv_proj_stage(dx, dws, None, targets=SPATIAL)
        cache.ca2_cache_commit()
        hk, hv, hks, hvs = cache.ca2_cache_debug_copy()
        _, kt, vt = (_split(t, sh, n) for t in qkv_proj_tpe_ref(x, wt, rows, fw, n, S))
        _, ksp, vsp = (_split(t, sh, n) for t in qkv_proj_tpe_ref(x, ws, 0 * rows, fw, n, S))
        for f in range(n):
            slot = (fw + f) % (P + l)
            check_close(bits_to_f32(hk[:, slot]), kt[:, f], "bf16", f"ring K frame {fw + f}")
            check_close(bits_to_f32(hv[:, slot]), vt[:, f], "bf16", f"ring V frame {fw + f}")
            if f >= n - Ps:
                ss = (fw + f) % Ps
                check_close(bits_to_f32(hks[:, ss]), ksp[:, f], "bf16", f"spatial K frame {fw + f}")
                check_close(bits_to_f32(hvs[:, ss]), vsp[:, f], "bf16", f"spatial V frame {fw + f}")
        fw += n
    cache.close()


def test_stage_state_errors_leave_the_cache_unchanged(ca2):
    sh = SMALL
    B, S, H, d, l = sh["B"], sh["S"], sh["H"], sh["d"], sh["l"]
    w, rows = _weights(sh, C_IN, 35)
    dw = to_dev(w, "bf16")
    dx = to_dev(_inputs(sh, C_IN, 11, l, 0), "bf16").view(B, l, S, C_IN)
    q = torch.zeros((B, l, S, H, d), dtype=torch.bfloat16, device="cuda")

    def status(fn):
        with pytest.raises(ca2.Ca2Error) as e:
            fn()
        return e.value.status

    plain = ca2.Cache.from_shape(sh)                         # no staging slots
    plain.ca2_cache_write(q, q, q, q)
    assert status(lambda: plain.ca2_qkv_proj_stage(dx, dw, targets=RING)) == ca2.CA2_ERR_STATE
    # the spatial buffer alone is refused too: the commit needs the ring, so it
    # would leave the cache with its prefix frames overwritten and no way out
    assert status(lambda: plain.ca2_qkv_proj_stage(dx, dw, targets=SPATIAL)) == ca2.CA2_ERR_STATE
    assert plain.ca2_cache_info_get()["staged_frames"] == 0
    plain.ca2_spatial_attn(q, q, q, q)                        # prefix mode still works
    assert status(lambda: plain.ca2_cache_commit()) == ca2.CA2_ERR_STATE           # nothing staged
    plain.close()

    cache = ca2.Cache.from_shape(sh, staged=True)
    assert status(lambda: cache.ca2_cache_commit()) == ca2.CA2_ERR_STATE           # nothing staged
    assert status(lambda: cache.ca2_temporal_attn(q, None, None, q)) == ca2.CA2_ERR_INVALID_ARG
    cache.ca2_qkv_proj_stage(dx, dw, targets=RING | SPATIAL)
    before = cache.ca2_cache_info_get()
    assert status(lambda: cache.ca2_qkv_proj_stage(dx, dw, targets=RING)) == ca2.CA2_ERR_STATE
    assert status(lambda: cache.ca2_cache_write(q, q, q, q)) == ca2.CA2_ERR_STATE
    assert status(lambda: cache.ca2_temporal_attn(q[:, :2].contiguous(), None, None,
                                                  q[:, :2].contiguous())) == ca2.CA2_ERR_INVALID_ARG
    bad_x = torch.empty((B, l, S, 96), dtype=torch.bfloat16, device="cuda")
    bad_w = torch.empty((3 * H * d, 96), dtype=torch.bfloat16, device="cuda")
    assert status(lambda: cache.ca2_qkv_proj_stage(bad_x, bad_w, targets=RING)) == ca2.CA2_ERR_INVALID_ARG
    assert cache.ca2_cache_info_get() == before
    cache.ca2_cache_commit()
    assert cache.ca2_cache_info_get()["frames_written"] == l
    cache.close()

    f32 = ca2.Cache(1, 2, 64, 16, 4, 5, 1, 9, "f32", staged=True)
    x32 = torch.empty((1, 4, 16, 64), dtype=torch.bfloat16, device="cuda")
    w32 = torch.empty((384, 64), dtype=torch.bfloat16, device="cuda")
    assert status(lambda: f32.ca2_qkv_proj_stage(x32, w32, targets=RING)) == ca2.CA2_ERR_UNSUPPORTED
    f32.close()


def test_write_case_full_size_sampled(ca2):
    """The cache-writing workload (B4, chunk 8, 256 tokens, 16 x 72, P_max 41,
    P' 3, TPE table 49), started full so the commit evicts: sampled rows of the
    fused output against the oracle row by row, every staged ring / spatial
    frame bit-identical to the caller outputs, and the write-pass temporal
    attention read from the ring equal bitwise to the same call given the
    caller's K/V."""
    sh = synth.WORKLOADS["write_b4"]
    B, S, H, d, l, P, Ps, L = (sh[k] for k in ("B", "S", "H", "d", "l", "p_max", "p_spatial", "tpe_len"))
    C = H * d
    cache = ca2.Cache.from_shape(sh, staged=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    for n in [1] + [l] * 5:                              # 41 frames: the queue is full
        k0 = torch.randn((B, n, S, H, d), generator=gen, device="cuda").to(torch.bfloat16)
        cache.ca2_cache_write(k0, k0, k0, k0)
    fw = cache.ca2_cache_info_get()["frames_written"]
    assert fw == P
    x = synth.activations(40, B * l * S, C)
    w = synth.weight(40, 3 * C, C, 0.02)
    rows = synth.normal(40, "w", (4, L, 3 * C), (L, 3 * C), "f32", std=0.5)
    dq, dk, dv = (torch.empty((B, l, S, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    cache.ca2_qkv_proj_stage(to_dev(x, "bf16").view(B, l, S, C), to_dev(w, "bf16"),
                             torch.from_numpy(rows).cuda(), dq, dk, dv)
    out_ring, out_own = torch.empty_like(dq), torch.empty_like(dq)
    cache.ca2_temporal_attn(dq, None, None, out_ring)
    cache.ca2_temporal_attn(dq, dk, dv, out_own)
    torch.cuda.synchronize()
    assert torch.equal(out_ring.view(torch.int16), out_own.view(torch.int16))
    # sampled whole frames against the oracle, each as a one-frame chunk starting at its frame id
    got = np.concatenate([to_host(t.view(-1, C)) for t in (dq, dk, dv)], 1)
    for b, f in ((0, 0), (0, 7), (3, 2), (3, 7)):
        r0 = (b * l + f) * S
        ref = np.concatenate(qkv_proj_tpe_ref(x[r0:r0 + S], w, rows, fw + f, 1, S), 1)
        check_close(got[r0:r0 + S], ref, "bf16", f"batch {b} frame {f}")
    hk, hv, hks, hvs = cache.ca2_cache_debug_copy()
    kb = dk.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = dv.view(torch.int16).cpu().numpy().view(np.uint16)
    for f in range(l):
        slot = (fw + f) % (P + l)
        assert np.array_equal(hk[:, slot], kb[:, f]) and np.array_equal(hv[:, slot], vb[:, f])
        if f >= l - Ps:
            assert np.array_equal(hks[:, (fw + f) % Ps], kb[:, f])
            assert np.array_equal(hvs[:, (fw + f) % Ps], vb[:, f])
    cache.ca2_cache_commit()
    info = cache.ca2_cache_info_get()
    assert info["p_k"] == P and info["frames_written"] == P + l
    assert info["bytes_resident"] == 2 * B * (P + l + Ps) * S * C * 2
    cache.close()


@pytest.mark.parametrize("sh", [
    dict(B=1, H=1, d=128, S=70, l=3, p_max=4, p_spatial=0, tpe_len=7, dtype="bf16"),     # no spatial buffer
    dict(B=3, H=8, d=72, S=33, l=8, p_max=9, p_spatial=5, tpe_len=20, dtype="bf16"),     # C = 576, ragged tokens
], ids=["d128_no_prefix", "d72_ragged"])
def test_staged_other_shapes(ca2, sh):
    """Stage + write-pass temporal attention read from the ring + commit over
    writes that evict and wrap, against the oracle (projection with TPE,
    attention over the oracle's bf16 K/V); queue placement bit-exact."""
    B, S, H, d, l, P, Ps = sh["B"], sh["S"], sh["H"], sh["d"], sh["l"], sh["p_max"], sh["p_spatial"]
    c_in = 64
    cache = ca2.Cache.from_shape(sh, staged=True)
    w, rows = _weights(sh, c_in, 36)
    dw, drows = to_dev(w, "bf16"), torch.from_numpy(rows.astype(np.float32)).cuda()
    oq = TemporalQueue(P, slots=P + l)
    ok_frames, ov_frames = {}, {}
    fw = 0
    for step, n in enumerate([1, l, 2, l, l]):
        x = _inputs(sh, c_in, 12, n, step)
        exact = [_split(t, sh, n) for t in qkv_proj_tpe_ref(x, w, rows, fw, n, S)]
        q_ref, k_ref, v_ref = (_bf16(t) for t in exact)
        dq = torch.empty((B, n, S, H, d), dtype=torch.bfloat16, device="cuda")
        targets = RING | (SPATIAL if Ps else 0)
        cache.ca2_qkv_proj_stage(to_dev(x, "bf16").view(B, n, S, c_in), dw, drows, dq, None, None, targets=targets)
        out = torch.empty_like(dq)
        cache.ca2_temporal_attn(dq, None, None, out)
        torch.cuda.synchronize()
        check_close(to_host(dq), exact[0], "bf16", f"step {step} projected q")
        ids = oq.frame_ids()
        rk = np.stack([ok_frames[f] for f in ids], 1) if ids else np.zeros((B, 0, S, H, d))
        rv = np.stack([ov_frames[f] for f in ids], 1) if ids else np.zeros((B, 0, S, H, d))
        check_close(to_host(out), temporal_attn_ref(q_ref, k_ref, v_ref, rk, rv, list(range(len(ids))), d ** -0.5),
                    "bf16", f"step {step} write-pass temporal attention")
        hk, hv, _, _ = cache.ca2_cache_debug_copy()
        for f in range(n):
            slot = (fw + f) % (P + l)
            check_close(bits_to_f32(hk[:, slot]), exact[1][:, f], "bf16", f"ring K frame {fw + f}")
            check_close(bits_to_f32(hv[:, slot]), exact[2][:, f], "bf16", f"ring V frame {fw + f}")
        cache.ca2_cache_commit()
        oq.write(range(fw, fw + n))
        for f in range(n):
            ok_frames[fw + f], ov_frames[fw + f] = k_ref[:, f], v_ref[:, f]
        fw += n
        assert cache.ca2_cache_slot_map() == oq.slot_map()
    cache.close()


def test_random_mixed_write_paths(ca2):
    """Seeded random sequences on a cache with staging slots: each chunk (random
    size 1..l) goes in either by the copy path (ca2_cache_write) or by the fused
    stage + commit, so the two placements interleave through eviction and ring
    wrap. After every write the slot map equals the oracle queue's, and a
    denoising call's temporal and prefix spatial attention match the oracle
    over the oracle's own cached K/V."""
    sh = dict(B=1, H=2, d=64, S=24, l=4, p_max=6, p_spatial=2, tpe_len=10, dtype="bf16")
    B, S, H, d, l, P, Ps = sh["B"], sh["S"], sh["H"], sh["d"], sh["l"], sh["p_max"], sh["p_spatial"]
    c_in = 64
    rng = np.random.default_rng(99)
    w, rows = _weights(sh, c_in, 37)
    dw, drows = to_dev(w, "bf16"), torch.from_numpy(rows.astype(np.float32)).cuda()
    cache = ca2.Cache.from_shape(sh, staged=True)
    oq, osp = TemporalQueue(P, slots=P + l), SpatialCache(Ps)
    okf, ovf = {}, {}
    fw = 0
    for step in range(14):
        n = 1 if step == 0 else int(rng.integers(1, l + 1))
        if rng.random() < 0.5:
            x = _inputs(sh, c_in, 13, n, step)
            exact = [_split(t, sh, n) for t in qkv_proj_tpe_ref(x, w, rows, fw, n, S)]
            k_ref, v_ref = _bf16(exact[1]), _bf16(exact[2])
            cache.ca2_qkv_proj_stage(to_dev(x, "bf16").view(B, n, S, c_in), dw, drows)
            cache.ca2_cache_commit()
            path = "staged"
        else:
            k_ref = synth.frames_tensor(14, "kt", range(fw, fw + n), B, S, H, d, "bf16").astype(np.float64)
            v_ref = synth.frames_tensor(14, "vt", range(fw, fw + n), B, S, H, d, "bf16").astype(np.float64)
            dk, dv = to_dev(k_ref.astype(np.float32), "bf16"), to_dev(v_ref.astype(np.float32), "bf16")
            cache.ca2_cache_write(dk, dv, dk, dv)
            path = "copy"
        oq.write(range(fw, fw + n))
        osp.write(range(fw, fw + n))
        for f in range(n):
            okf[fw + f], ovf[fw + f] = k_ref[:, f], v_ref[:, f]
        fw += n
        assert cache.ca2_cache_slot_map() == oq.slot_map(), f"step {step} ({path})"
        q, k, v = (synth.step_tensor(15, nm, step, 0, B, l, S, H, d, "bf16") for nm in ("q", "k", "v"))
        dq, dk, dv = (to_dev(t, "bf16") for t in (q, k, v))
        ot, os_ = torch.empty_like(dq), torch.empty_like(dq)
        cache.ca2_temporal_attn(dq, dk, dv, ot)
        cache.ca2_spatial_attn(dq, dk, dv, os_)
        torch.cuda.synchronize()
        ids = oq.frame_ids()
        rk, rv = np.stack([okf[f] for f in ids], 1), np.stack([ovf[f] for f in ids], 1)
        check_close(to_host(ot), temporal_attn_ref(q, k, v, rk, rv, list(range(len(ids))), d ** -0.5), "bf16",
                    f"step {step} ({path}) temporal")
        pf = osp.logical_frames()
        ks, vs = np.stack([okf[f] for f in pf], 1), np.stack([ovf[f] for f in pf], 1)
        check_close(to_host(os_), spatial_attn_ref(q, k, v, ks, vs, list(range(Ps)), d ** -0.5, "prefix"), "bf16",
                    f"step {step} ({path}) spatial")
    cache.close()
