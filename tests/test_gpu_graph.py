"""HIP-graph capture of the denoising loop (the calls that share one cache
state between two cache-writing passes), checked against the oracle.

The loop is captured once and replayed several times, with the program's own
eager launches and synchronisations between replays. Every replay's outputs
are compared element by element with the oracle's prefix spatial and causal
temporal attention over the same cache state (bf16 bar), and must also be
bit-identical to eager launches of the same calls (the kernels are
deterministic: no atomics, fixed reduction order). The cache's state
generation is read at capture and must be unchanged at every replay (the
graph's baked-in queue state is current).
"""
import pytest
import torch

from oracle import RolloutOracle, temporal_attn_ref
from gpu_util import to_dev, to_host, check_close

pytestmark = pytest.mark.gpu

# the 256-token Ca2-VDM shape of the benchmark step, queue full
SHAPE = dict(B=1, H=16, d=72, S=256, l=8, p_max=25, p_spatial=3, tpe_len=33, dtype="bf16")
CALLS = 4


def test_denoise_loop_graph_replays_match_oracle(ca2):
    sh = SHAPE
    cache = ca2.Cache.from_shape(sh)
    o = RolloutOracle(sh, 2024)
    for w in (1, 8, 8, 8):                           # queue and spatial cache full
        frames = o.next_frames(w)
        cache.ca2_cache_write(*(to_dev(o.clean(x, frames), "bf16") for x in ("kt", "vt", "ks", "vs")))
        o.write(frames)
    n = sh["l"]
    host = [tuple(o.noisy(x, 1, t, n) for x in ("q", "k", "v")) for t in range(CALLS)]
    sets = [tuple(to_dev(x, "bf16") for x in qkv) for qkv in host]
    outs = [(torch.empty_like(q), torch.empty_like(q)) for q, _, _ in sets]
    refs = []
    for q, k, v in host:
        refs.append((o.spatial_out(q, k, v, "prefix"),
                     temporal_attn_ref(q, k, v, o.ring_k, o.ring_v, o.queue.slot_map(), o.scale)))

    def loop():
        for (q, k, v), (os_, ot) in zip(sets, outs):
            cache.ca2_spatial_attn(q, k, v, os_)
            cache.ca2_temporal_attn(q, k, v, ot)

    def check_oracle(tag):
        for i, ((a, b), (rs, rt)) in enumerate(zip(outs, refs)):
            check_close(to_host(a), rs, "bf16", f"{tag}: spatial call {i}")
            check_close(to_host(b), rt, "bf16", f"{tag}: temporal call {i}")

    loop()
    torch.cuda.synchronize()
    check_oracle("eager")
    eager = [(a.clone(), b.clone()) for a, b in outs]

    gen = cache.ca2_cache_info_get()["generation"]
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
        assert cache.ca2_cache_info_get()["generation"] == gen
        g.replay()
        torch.cuda.synchronize()
        check_oracle(f"replay {rep}")
        for i, ((a, b), (ea, eb)) in enumerate(zip(outs, eager)):
            assert torch.equal(a, ea), f"replay {rep}: spatial output of call {i} differs from eager"
            assert torch.equal(b, eb), f"replay {rep}: temporal output of call {i} differs from eager"
        loop()                                       # eager work between replays
        torch.cuda.synchronize()
        for (a, b), (ea, eb) in zip(outs, eager):
            assert torch.equal(a, ea) and torch.equal(b, eb), "eager launch after a replay differs"
    del g
    cache.close()
