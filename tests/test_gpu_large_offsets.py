"""A cache whose ring spans more than 4 GiB (64x64-latent frames of 4096
tokens x 16 heads x 72, P_max = 480 queued frames: 9.1 GB of K/V), filled
past eviction and wrap, so the cache write and both attention kernels run
with byte offsets beyond 32 bits. Inputs are seeded torch draws made on the
device; the oracle checks sampled rows (temporal) and sampled queries
(spatial) from host copies of exactly those inputs. bf16 bar: max-abs 2e-2."""
import numpy as np
import pytest
import torch

from oracle import temporal_attn_ref, spatial_attn_ref
from gpu_util import to_dev, to_host, check_close

pytestmark = pytest.mark.gpu

B, H, d, S, L, P_MAX, P_SP = 1, 16, 72, 4096, 8, 480, 3


def test_ring_beyond_4gib(ca2):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260)
    cache = ca2.Cache(B, H, d, S, L, P_MAX, P_SP, P_MAX + L, "bf16")
    assert cache.ca2_cache_info_get()["bytes_resident"] > 2 ** 33
    rng = np.random.default_rng(7)
    rows = [(int(s), int(h)) for s, h in zip(rng.integers(0, S, 24), rng.integers(0, H, 24))]
    s_idx = torch.tensor([r[0] for r in rows], device="cuda")
    h_idx = torch.tensor([r[1] for r in rows], device="cuda")

    def draw(n):
        return [torch.randn((B, n, S, H, d), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(4)]

    def rows_of(t):          # [B][n][S][H][d] -> host [B][n][R][d] at the sampled (s, h)
        return to_host(t[:, :, s_idx, h_idx])

    kt_hist, vt_hist = [], []  # sampled temporal K/V of every written frame, in order
    spatial_last = None        # full spatial K/V of the last chunk (the buffer holds its last P' frames)
    for n in [1] + [L] * 60:   # 481 frames: the queue holds frames 1..480, the ring has wrapped
        kt, vt, ks, vs = draw(n)
        cache.ca2_cache_write(kt, vt, ks, vs)
        kt_hist.append(rows_of(kt))
        vt_hist.append(rows_of(vt))
        spatial_last = (ks, vs)
    torch.cuda.synchronize()
    info = cache.ca2_cache_info_get()
    assert info["p_k"] == P_MAX and info["frames_written"] == 481
    q, k, v = (torch.randn((B, L, S, H, d), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
    out_t = torch.empty_like(q)
    out_s = torch.empty_like(q)
    cache.ca2_temporal_attn(q, k, v, out_t)
    cache.ca2_spatial_attn(q, k, v, out_s)
    torch.cuda.synchronize()

    # temporal: sampled rows against the oracle over the queued frames 1..480
    kq = np.concatenate(kt_hist, axis=1)[:, 1:]            # [B][480][R][d]
    vq = np.concatenate(vt_hist, axis=1)[:, 1:]
    R = len(rows)
    ring_k = kq.reshape(B, P_MAX, R, 1, d)                  # the queue in logical order, one row per "token"
    ring_v = vq.reshape(B, P_MAX, R, 1, d)
    ref = temporal_attn_ref(rows_of(q).reshape(B, L, R, 1, d), rows_of(k).reshape(B, L, R, 1, d),
                            rows_of(v).reshape(B, L, R, 1, d), ring_k, ring_v, list(range(P_MAX)), d ** -0.5)
    check_close(rows_of(out_t).reshape(B, L, R, 1, d), ref, "bf16", "temporal, 9.1 GB ring")

    # spatial: sampled queries of two (frame, head) pairs; prefix = the last P' clean frames
    ks, vs = spatial_last
    ks_h, vs_h = to_host(ks[:, -P_SP:]), to_host(vs[:, -P_SP:])   # frames 478..480, oldest first
    qh, kh, vh, oh = to_host(q), to_host(k), to_host(v), to_host(out_s)
    toks = np.sort(rng.choice(S, 48, replace=False))
    for f, h in ((0, 3), (7, 15)):
        sl = (slice(None), slice(f, f + 1))
        ref_s = spatial_attn_ref(qh[sl][:, :, toks][:, :, :, h:h + 1], kh[sl][:, :, :, h:h + 1],
                                 vh[sl][:, :, :, h:h + 1], ks_h[:, :, :, h:h + 1], vs_h[:, :, :, h:h + 1],
                                 list(range(P_SP)), d ** -0.5, "prefix")
        check_close(oh[sl][:, :, toks][:, :, :, h:h + 1], ref_s, "bf16", f"spatial frame {f} head {h}")
    cache.close()


def test_staged_write_beyond_4gib(ca2):
    """The fused cache-writing stage on a ring of 488 slots (9.2 GB of K/V):
    after 481 frames the next chunk's slots start 4.5 GB into the ring, so
    the epilogue's ring offsets are beyond 32 bits. The write-pass temporal
    attention reading the staged frames from those slots must equal, bit for
    bit, the same call given the caller's K/V outputs; sampled projection rows
    match the oracle (bf16 bar)."""
    from oracle import qkv_proj_tpe_ref
    import synth
    C = H * d
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261)
    cache = ca2.Cache(B, H, d, S, L, P_MAX, P_SP, P_MAX + L, "bf16", staged=True)
    info = cache.ca2_cache_info_get()
    assert info["ring_slots"] == P_MAX + L and info["bytes_resident"] > 2 ** 33
    for n in [1] + [L] * 60:
        t = torch.randn((B, n, S, H, d), generator=gen, device="cuda").to(torch.bfloat16)
        cache.ca2_cache_write(t, t, t, t)
    fw = cache.ca2_cache_info_get()["frames_written"]
    assert fw == 481
    frame_bytes = S * C * 2
    assert (fw % (P_MAX + L)) * frame_bytes > 2 ** 32          # the staged slots lie past 4 GiB
    x = synth.normal(5, "x", (3, 9, 1, L, S, 64), (B * L * S, 64), "bf16")
    w = synth.weight(5, 3 * C, 64, 0.05)
    rows = synth.normal(5, "w", (4, P_MAX + L, 3 * C), (P_MAX + L, 3 * C), "f32", std=0.5)
    dq, dk, dv = (torch.empty((B, L, S, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    cache.ca2_qkv_proj_stage(to_dev(x, "bf16").view(B, L, S, 64), to_dev(w, "bf16"),
                             torch.from_numpy(rows).cuda(), dq, dk, dv)
    out_ring, out_own = torch.empty_like(dq), torch.empty_like(dq)
    cache.ca2_temporal_attn(dq, None, None, out_ring)
    cache.ca2_temporal_attn(dq, dk, dv, out_own)
    torch.cuda.synchronize()
    assert torch.equal(out_ring.view(torch.int16), out_own.view(torch.int16))
    got = torch.cat([t.view(-1, C) for t in (dq, dk, dv)], 1)
    for f in (0, 7):
        r0 = f * S + 1000                                         # 48 tokens of frame f
        ref = np.concatenate(qkv_proj_tpe_ref(x[r0:r0 + 48], w, rows, fw + f, 1, 48), 1)
        check_close(to_host(got[r0:r0 + 48]), ref, "bf16", f"frame {f} rows")
    cache.ca2_cache_commit()
    info = cache.ca2_cache_info_get()
    assert info["p_k"] == P_MAX and info["frames_written"] == fw + L
    cache.close()
