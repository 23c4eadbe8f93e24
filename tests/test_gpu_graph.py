"""HIP-graph capture of the denoising loop (the calls that share one cache
state between two cache-writing passes).

The loop is captured once and replayed several times, with the program's own
eager launches and synchronisations between replays; every replay must give
outputs bit-identical to eager launches of the same calls (the kernels are
deterministic: no atomics, fixed reduction order).
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

SHAPE = dict(B=1, H=16, d=72, S=256, l=8, p_max=25, p_spatial=3, tpe_len=33)


def test_denoise_loop_graph_replays_equal_eager(ca2):
    sh = SHAPE
    bf = torch.bfloat16
    cache = ca2.Cache(sh["B"], sh["H"], sh["d"], sh["S"], sh["l"], sh["p_max"], sh["p_spatial"], sh["tpe_len"], "bf16")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    B, l, S, H, d = sh["B"], sh["l"], sh["S"], sh["H"], sh["d"]

    def randn(n):
        return torch.randn((B, n, S, H, d), generator=gen, device="cuda", dtype=torch.float32).to(bf)

    frames = 0
    while frames < sh["p_max"]:                      # queue full, spatial cache full
        n = 1 if frames == 0 else l
        cache.ca2_cache_write(randn(n), randn(n), randn(n), randn(n))
        frames += n
    T = 10
    sets = [(randn(l), randn(l), randn(l)) for _ in range(T)]
    outs = [(torch.empty_like(q), torch.empty_like(q)) for q, _, _ in sets]

    def loop():
        for (q, k, v), (os_, ot) in zip(sets, outs):
            cache.ca2_spatial_attn(q, k, v, os_)
            cache.ca2_temporal_attn(q, k, v, ot)

    loop()
    torch.cuda.synchronize()
    ref = [(a.clone(), b.clone()) for a, b in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        loop()
    torch.cuda.synchronize()

    for rep in range(3):
        for a, b in outs:
            a.zero_()
            b.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((a, b), (ra, rb)) in enumerate(zip(outs, ref)):
            assert torch.equal(a, ra), f"replay {rep}: spatial output of call {i} differs from eager"
            assert torch.equal(b, rb), f"replay {rep}: temporal output of call {i} differs from eager"
        loop()                                       # eager work between replays
        torch.cuda.synchronize()
        for (a, b), (ra, rb) in zip(outs, ref):
            assert torch.equal(a, ra) and torch.equal(b, rb), "eager launch after a replay differs"
