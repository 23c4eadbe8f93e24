"""GPU QKV projection (K4) against the oracle, then its K/V into the cache."""
import numpy as np
import pytest
import torch

import synth
from oracle import qkv_proj_ref
from gpu_util import to_dev, to_host, check_close

pytestmark = pytest.mark.gpu


def _run(ca2, m, c_in, c, seed):
    x = synth.activations(seed, m, c_in)
    w = synth.weight(seed, 3 * c, c_in, 0.02)
    dq, dk, dv = (torch.empty((m, c), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    ca2.ca2_qkv_proj(to_dev(x, "bf16"), to_dev(w, "bf16"), dq, dk, dv)
    torch.cuda.synchronize()
    return x, w, (dq, dk, dv)


@pytest.mark.parametrize("m,c_in,c", [(200, 128, 64), (131, 64, 192), (256, 1152, 1152)])
def test_qkv_small_ragged(ca2, m, c_in, c):
    x, w, outs = _run(ca2, m, c_in, c, 1)
    for got, ref, nm in zip(outs, qkv_proj_ref(x, w), "qkv"):
        check_close(to_host(got), ref, "bf16", f"qkv {nm} {m}x{c_in}x{c}")


def test_qkv_write_case_full_and_cache(ca2):
    """Cache-write workload: B=4 x l=8 x 256 tokens = 8192 rows, 1152 -> 3x1152."""
    sh = synth.WORKLOADS["write_b4"]
    B, l, S, H, d = sh["B"], sh["l"], sh["S"], sh["H"], sh["d"]
    m, c = B * l * S, H * d
    x, w, (dq, dk, dv) = _run(ca2, m, c, c, 2)
    refs = qkv_proj_ref(x, w)
    for got, ref, nm in zip((dq, dk, dv), refs, "qkv"):
        check_close(to_host(got), ref, "bf16", f"qkv {nm} full")
    # the projected K/V of the clean chunk go into a cache as [B][l][S][H][d]
    cache = ca2.Cache.from_shape(sh)
    kk = dk.view(B, l, S, H, d)
    vv = dv.view(B, l, S, H, d)
    cache.ca2_cache_write(kk, vv, kk, vv)
    ring_k = cache.ca2_cache_debug_copy()[0]
    got = ring_k[:, :8]                     # frames 0..7 -> slots 0..7
    assert np.array_equal(got, dk.view(torch.int16).cpu().numpy().view(np.uint16).reshape(B, l, S, H, d))
