"""Benchmark of the shared-cache attention hot path on one MI355X.

A step is one autoregressive step at the 256-token Ca2-VDM shape (B=1, 16
heads x 72, 16x16 latent tokens, chunk l=8, queue full at P_max=25, P'=3,
bf16): 50 denoising calls -- each a prefix-enhanced spatial attention and a
causal temporal attention over the shared cache, with fresh Q/K/V per call,
computed by one fused launch (ca2_denoise_attn) -- then the cache-writing
pass: spatial self attention, temporal attention of the clean chunk, and the
cache write (append + FIFO evict + spatial overwrite).
Inputs are synthetic (seeded N(0,1), bf16) and resident in HBM before timing.

value = denoising-call query tokens (50 * B*l*S per step) / wall time of the
whole step (the cache-writing pass is timed but its tokens are not counted).

Also reported: per-kernel average duration from HIP events on the launch
stream, the dominant kernel's roofline fraction, the batched 32x32-latent
case (B=8, 1024 tokens) whose temporal working set (1.5 GB) exceeds the
256 MB Infinity Cache, the 80-frame rollout through the cached path against
the recompute baseline (bidirectional temporal + spatial self attention over
all conditional frames at every call), and the CPU oracle timed on a bounded
sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-large] [--no-rollout]
       python bench.py --kernel {spatial_prefix,temporal,spatial_self,cache_write,qkv_proj,qkv_proj_stage}
                       --workload {ar_step_s256,large_b8_s1024,write_b4} --reps R   (one kernel, for profilers)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention tokens/sec per denoise step; temporal HBM GB/s, spatial MFMA util %"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure
T_DENOISE = 50
N_CACHES = 8      # per-layer caches rotated through at the 256-token shape

AR_STEP = dict(name="ar_step_s256", B=1, H=16, d=72, S=256, l=8, p_max=25, p_spatial=3, tpe_len=33)
LARGE = dict(name="large_b8_s1024", B=8, H=16, d=72, S=1024, l=8, p_max=25, p_spatial=3, tpe_len=33)
WRITE = dict(name="write_b4", B=4, H=16, d=72, S=256, l=8, p_max=41, p_spatial=3, tpe_len=49)
ROLLOUT = dict(name="rollout_80f", B=1, H=16, d=72, S=256, l=8, p_max=41, p_spatial=3, tpe_len=49)
ROLLOUT_FRAMES = 80
ROLLOUT_LAYERS = 8   # attention layers per model call in the rollout comparison
WORKLOADS = {w["name"]: w for w in (AR_STEP, LARGE, WRITE)}
KERNELS = ("spatial_prefix", "temporal", "spatial_self", "cache_write", "qkv_proj", "qkv_proj_stage",
           "denoise_fused")


# ----------------------------------------------------------------------------
# algorithmic work per launch
# ----------------------------------------------------------------------------
def temporal_bytes(sh, n, p_k, eb=2):
    C = sh["H"] * sh["d"]
    tok = sh["B"] * sh["S"] * C * eb
    return 2 * n * tok + 2 * p_k * tok + 2 * n * tok      # Q + O, cached K/V, new K/V


def temporal_flops(sh, n, p_k):
    rows = sh["B"] * sh["S"] * sh["H"]
    return rows * sum(p_k + i + 1 for i in range(n)) * 4 * sh["d"]


def spatial_flops(sh, n, n_prefix):
    S = sh["S"]
    return sh["B"] * n * sh["H"] * 4 * S * (n_prefix + 1) * S * sh["d"]


def spatial_bytes(sh, n, n_prefix, eb=2):
    C = sh["H"] * sh["d"]
    tok = sh["B"] * sh["S"] * C * eb
    return 4 * n * tok + 2 * n_prefix * tok                # Q, O, own K, V; prefix K/V read once


def write_bytes(sh, n, eb=2):
    C = sh["H"] * sh["d"]
    tok = sh["B"] * sh["S"] * C * eb
    return 2 * (2 * n * tok + 2 * min(n, sh["p_spatial"]) * tok)   # read + write of K/V copies


# ----------------------------------------------------------------------------
def _randn(shape, gen, dtype):
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(dtype)


class Workload:
    """Device buffers and `n_caches` caches filled to P_max for one shape.

    Several caches stand for the per-layer caches of a model: consecutive
    denoising calls use consecutive caches, and each cache-writing pass writes
    the next one, so the rotated working set (caches plus Q/K/V sets) exceeds
    the 256 MB Infinity Cache and the temporal reads are served by HBM."""

    def __init__(self, sh, n_sets, seed, n_caches=1):
        import torch
        from causal_kv_cache_amd import ca2
        self.sh = sh
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        bf = torch.bfloat16
        B, l, S, H, d = sh["B"], sh["l"], sh["S"], sh["H"], sh["d"]
        chunk = (B, l, S, H, d)
        self.caches = []
        for _ in range(n_caches):
            c = ca2.Cache(B, H, d, S, l, sh["p_max"], sh["p_spatial"], sh["tpe_len"], "bf16")
            # fill the queue: conditioning frame, then whole chunks, to P_max frames
            frames = 0
            while frames < sh["p_max"]:
                w = 1 if frames == 0 else l
                t = [_randn((B, w, S, H, d), gen, bf) for _ in range(4)]
                c.ca2_cache_write(*t)
                frames += w
            self.caches.append(c)
        self.cache = self.caches[0]
        self.sets = [tuple(_randn(chunk, gen, bf) for _ in range(3)) for _ in range(n_sets)]
        self.clean = tuple(_randn(chunk, gen, bf) for _ in range(5))   # qc, kt, vt, ks, vs
        self.out_t = torch.empty(chunk, dtype=bf, device="cuda")
        self.out_s = torch.empty(chunk, dtype=bf, device="cuda")
        self.passes = 0
        torch.cuda.synchronize()

    def temporal_set(self, i):
        """The temporal layer's Q/K/V of call i: another set than the spatial
        layer's, so the two halves of a call read independent tensors."""
        return self.sets[(i + len(self.sets) // 2) % len(self.sets)]

    def denoise(self, i):
        """One denoising call: prefix spatial + causal temporal attention over
        one cache, fused into one launch where the shapes allow it."""
        q, k, v = self.sets[i % len(self.sets)]
        qt, kt, vt = self.temporal_set(i)
        c = self.caches[i % len(self.caches)]
        c.ca2_denoise_attn(q, k, v, self.out_s, qt, kt, vt, self.out_t)

    def denoise_two_launches(self, i):
        """The same call as two launches (stand-alone spatial, then temporal)."""
        q, k, v = self.sets[i % len(self.sets)]
        qt, kt, vt = self.temporal_set(i)
        c = self.caches[i % len(self.caches)]
        c.ca2_spatial_attn(q, k, v, self.out_s)
        c.ca2_temporal_attn(qt, kt, vt, self.out_t)

    def write_pass(self):
        from causal_kv_cache_amd import ca2
        qc, kt, vt, ks, vs = self.clean
        c = self.caches[self.passes % len(self.caches)]
        self.passes += 1
        c.ca2_tpe_index(self.sh["l"])
        # the pass's spatial (self mode) and temporal attention in one launch
        c.ca2_denoise_attn(qc, ks, vs, self.out_s, qc, kt, vt, self.out_t, mode=ca2.CA2_SPATIAL_SELF)
        c.ca2_cache_write(kt, vt, ks, vs)

    def ar_step(self):
        for t in range(T_DENOISE):
            self.denoise(t)
        self.write_pass()


def time_launches_stats(fn, reps, rounds=5):
    """Per-launch duration of `fn` in microseconds: `rounds` blocks of `reps`
    back-to-back launches, each block timed with HIP events recorded on the
    current (launch) stream; returns (median, min, max) of the block averages."""
    import statistics
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    vals = []
    for _ in range(rounds):
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        vals.append(e0.elapsed_time(e1) * 1e3 / reps)
    return statistics.median(vals), min(vals), max(vals)


def time_launches(fn, reps, rounds=5):
    """Median per-launch duration (microseconds) over `rounds` blocks of `reps` launches."""
    return time_launches_stats(fn, reps, rounds)[0]


def denoise_loop_graph(w: Workload, reps: int):
    """The 50 denoising calls of one AR step (they share one state of each
    cache) launched eagerly as fused calls, eagerly as two launches per call,
    and as one captured HIP graph of the fused calls: average ms per loop.
    The cache-writing pass changes the queue and cannot be replayed, so the
    headline step launches eagerly; this only reports the difference."""
    import torch

    def loop():
        for t in range(T_DENOISE):
            w.denoise(t)

    def loop2():
        for t in range(T_DENOISE):
            w.denoise_two_launches(t)

    eager = time_launches(loop, reps) / 1e3
    two = time_launches(loop2, reps) / 1e3
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        loop()
    torch.cuda.synchronize()
    graph = time_launches(g.replay, reps) / 1e3
    del g
    return eager, two, graph


def launchers(w: Workload):
    """One launch of each attention kernel, rotating through the workload's
    caches and Q/K/V sets as consecutive denoising calls do."""
    from causal_kv_cache_amd import ca2
    sets, caches = w.sets, w.caches
    idx = [0]

    def nxt():
        idx[0] += 1
        return caches[idx[0] % len(caches)], sets[idx[0] % len(sets)]

    def k_spatial():
        c, (q, k, v) = nxt()
        c.ca2_spatial_attn(q, k, v, w.out_s)

    def k_temporal():
        c, (q, k, v) = nxt()
        c.ca2_temporal_attn(q, k, v, w.out_t)

    def k_spatial_self():
        c, _ = nxt()
        qc, kt, vt, ks, vs = w.clean
        c.ca2_spatial_attn(qc, ks, vs, w.out_s, mode=ca2.CA2_SPATIAL_SELF)

    def k_denoise_fused():
        c, (q, k, v) = nxt()
        qt, kt, vt = w.temporal_set(idx[0])
        c.ca2_denoise_attn(q, k, v, w.out_s, qt, kt, vt, w.out_t)

    return {"spatial_prefix": k_spatial, "temporal": k_temporal, "spatial_self": k_spatial_self,
            "denoise_fused": k_denoise_fused}


def main_workload():
    """The headline workload: the 256-token shape with 8 rotating caches and
    one Q/K/V set per denoising call."""
    return Workload(AR_STEP, T_DENOISE, seed=1234, n_caches=N_CACHES)


def kernel_table(w: Workload, reps: int, fused: bool = False):
    """Per-kernel average launch duration and roofline numbers for one workload
    (with fused = True also the fused denoising call)."""
    sh = w.sh
    n, pk, ps = sh["l"], sh["p_max"], sh["p_spatial"]
    fns = launchers(w)
    k_spatial, k_temporal, k_spatial_self = fns["spatial_prefix"], fns["temporal"], fns["spatial_self"]

    rows = {}
    us, lo, hi = time_launches_stats(k_spatial, reps)
    fl = spatial_flops(sh, n, ps)
    rows["spatial_attn_prefix"] = dict(us=us, us_min=lo, us_max=hi, flops=fl, bytes=spatial_bytes(sh, n, ps),
                                       bound="mfma", achieved=fl / us / 1e6, peak=MFMA_BF16_PEAK_TFLOPS,
                                       unit="TFLOP/s")
    us, lo, hi = time_launches_stats(k_temporal, reps)
    by = temporal_bytes(sh, n, pk)
    rows["temporal_attn"] = dict(us=us, us_min=lo, us_max=hi, flops=temporal_flops(sh, n, pk), bytes=by,
                                 bound="hbm", achieved=by / us / 1e3, peak=HBM_PEAK_GBS, unit="GB/s")
    # the other bf16 temporal kernel (whole rows on the matrix cores), for comparison
    from causal_kv_cache_amd import ca2
    ca2.ca2_set_temporal_variant(2)
    try:
        us, lo, hi = time_launches_stats(k_temporal, reps)
    finally:
        ca2.ca2_set_temporal_variant(0)
    rows["temporal_attn_mfma_rows"] = dict(us=us, us_min=lo, us_max=hi, flops=temporal_flops(sh, n, pk), bytes=by,
                                           bound="hbm", achieved=by / us / 1e3, peak=HBM_PEAK_GBS, unit="GB/s")
    us, lo, hi = time_launches_stats(k_spatial_self, max(4, reps // 4))
    fl = spatial_flops(sh, n, 0)
    rows["spatial_attn_self"] = dict(us=us, us_min=lo, us_max=hi, flops=fl, bytes=spatial_bytes(sh, n, 0),
                                     bound="mfma", achieved=fl / us / 1e6, peak=MFMA_BF16_PEAK_TFLOPS,
                                     unit="TFLOP/s")
    if fused:
        # one launch doing both: its roofline is the larger of the two ideal
        # times of its combined work (bytes at HBM peak, flops at MFMA peak)
        us, lo, hi = time_launches_stats(fns["denoise_fused"], reps)
        fl = spatial_flops(sh, n, ps) + temporal_flops(sh, n, pk)
        by = spatial_bytes(sh, n, ps) + temporal_bytes(sh, n, pk)
        hbm_bound = by / HBM_PEAK_GBS >= fl / MFMA_BF16_PEAK_TFLOPS / 1e3
        rows["denoise_fused"] = dict(us=us, us_min=lo, us_max=hi, flops=fl, bytes=by,
                                     bound="hbm" if hbm_bound else "mfma",
                                     achieved=by / us / 1e3 if hbm_bound else fl / us / 1e6,
                                     peak=HBM_PEAK_GBS if hbm_bound else MFMA_BF16_PEAK_TFLOPS,
                                     unit="GB/s" if hbm_bound else "TFLOP/s",
                                     mfma_part={"achieved_tflops": round(fl / us / 1e6, 3),
                                                "frac": round(fl / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)},
                                     hbm_part={"achieved_gbs": round(by / us / 1e3, 3),
                                               "frac": round(by / us / 1e3 / HBM_PEAK_GBS, 4)})
    for r in rows.values():
        r["frac"] = r["achieved"] / r["peak"]
    return rows


SOURCES = {"spatial_prefix": "spatial_attn.hip", "spatial_self": "spatial_attn.hip",
           "denoise_fused": "spatial_attn.hip",
           "temporal": "temporal_attn.hip", "cache_write": "cache_write.hip", "qkv_proj": "qkv_proj.hip",
           "qkv_proj_stage": "qkv_proj.hip"}


def source_hash(kernel):
    """Hash of the kernel's source file and the library headers it includes
    (directly or through other headers), with comments and whitespace removed
    (a comment edit does not invalidate recorded counters)."""
    import re
    csrc = os.path.join(ROOT, "causal_kv_cache_amd", "csrc")
    names, todo = [], [SOURCES[kernel]]
    while todo:
        name = todo.pop(0)
        if name in names or not os.path.exists(os.path.join(csrc, name)):
            continue
        names.append(name)
        with open(os.path.join(csrc, name)) as f:
            todo += re.findall(r'#include\s+"([^"]+)"', f.read())
    src = ""
    for name in names:
        with open(os.path.join(csrc, name)) as f:
            src += f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"\s+", "", src)
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (profiles/traffic.json, already scaled by the copy-kernel calibration),
    or None when missing or when the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    e = t.get("kernels", {}).get(f"{kernel}@{workload}")
    if not e or e.get("source_sha256_16") != source_hash(kernel):
        return None
    return e.get("hbm_bytes_per_launch")


def write_case(reps, rounds=5, only=None):
    """Cache-writing stage at write_b4: QKV projection of the clean chunk
    (B*l*S x 1152 -> 3 x 1152) and the cache write of its K/V, then the same
    stage fused (ca2_qkv_proj_stage on a cache with staging slots: Q to the
    caller, K/V straight into the ring slots and the spatial buffer, the
    projected TPE row added, and the commit). The queue starts full, so every
    write evicts. only = "qkv_proj" or "qkv_proj_stage" times just that one
    (profiling)."""
    import torch
    from causal_kv_cache_amd import ca2
    sh = WRITE
    B, l, S, H, d = sh["B"], sh["l"], sh["S"], sh["H"], sh["d"]
    m, c = B * l * S, H * d
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    x = _randn((m, c), gen, torch.bfloat16)
    wgt = (torch.randn((3 * c, c), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    q, k, v = (torch.empty((m, c), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    w = Workload(sh, 1, seed=8)
    kk, vv = k.view(B, l, S, H, d), v.view(B, l, S, H, d)
    fl = 2 * m * c * 3 * c
    # the staged cache, filled to P_max
    st = ca2.Cache(B, H, d, S, l, sh["p_max"], sh["p_spatial"], sh["tpe_len"], "bf16", staged=True)
    f1 = kk[:, :1].contiguous()
    st.ca2_cache_write(f1, f1, f1, f1)
    while st.ca2_cache_info_get()["p_k"] < sh["p_max"]:
        st.ca2_cache_write(kk, vv, kk, vv)
    tpe = (torch.randn((sh["tpe_len"], 3 * c), generator=gen, device="cuda") * 0.02).contiguous()
    x4, q5 = x.view(B, l, S, c), q.view(B, l, S, H, d)

    def fused():
        st.ca2_qkv_proj_stage(x4, wgt, tpe, q5, None, None)
        st.ca2_cache_commit()

    if only == "qkv_proj_stage":
        us_f = time_launches(fused, reps, rounds)
        return {"qkv_proj_stage": {"us": round(us_f, 3), "flops": fl}}
    us_p = time_launches(lambda: ca2.ca2_qkv_proj(x, wgt, q, k, v), reps, rounds)
    if only == "qkv_proj":
        return {"qkv_proj": {"us": round(us_p, 3), "flops": fl}}
    us_w = time_launches(lambda: w.cache.ca2_cache_write(kk, vv, kk, vv), reps, rounds)
    us_f = time_launches(fused, reps, rounds)
    wb = write_bytes(sh, l)
    shared = w.cache.ca2_cache_info_get()["bytes_resident"]
    return {"workload": sh["name"],
            "qkv_proj": {"us": round(us_p, 3), "flops": fl, "achieved_tflops": round(fl / us_p / 1e6, 2),
                         "frac_mfma": round(fl / us_p / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_for("qkv_proj", sh["name"])},
            "cache_write": {"us": round(us_w, 3), "bytes": wb, "achieved_gbs": round(wb / us_w / 1e3, 1),
                            "frac_hbm": round(wb / us_w / 1e3 / HBM_PEAK_GBS, 4),
                            "traffic": traffic_for("cache_write", sh["name"])},
            "qkv_proj_stage_fused": {"us": round(us_f, 3), "unfused_us": round(us_p + us_w, 3),
                                     "achieved_tflops": round(fl / us_f / 1e6, 2),
                                     "frac_mfma": round(fl / us_f / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                                     "traffic": traffic_for("qkv_proj_stage", sh["name"])},
            "bytes_resident": {"shared_cache": shared, "per_timestep_copies_T50": 50 * shared,
                               "with_staging_slots": st.ca2_cache_info_get()["bytes_resident"]}}


def recompute_bytes(sh, T, eb=2):
    C = sh["H"] * sh["d"]
    return 4 * T * sh["B"] * sh["S"] * C * eb              # Q, K, V read once, O written


def recompute_temporal_flops(sh, T):
    return sh["B"] * sh["S"] * sh["H"] * T * T * 4 * sh["d"]


def rollout_compare():
    """80-frame rollout (B=1, 256 tokens, 16 heads x 72, chunk 8, P_max 41,
    P' 3, bf16) through the attention layers of an 8-layer model: the cached
    path (each AR step: 50 denoising calls of prefix spatial + causal temporal
    attention over the shared cache, then every layer's cache-writing pass)
    against the recompute baseline (each AR step: 50 calls of spatial self
    attention and bidirectional temporal attention over all P_k + 8 frames,
    no cache). GPU time per AR step from HIP events on the launch stream."""
    import torch
    from causal_kv_cache_amd import ca2
    sh, L = ROLLOUT, ROLLOUT_LAYERS
    B, l, S, H, d = sh["B"], sh["l"], sh["S"], sh["H"], sh["d"]
    bf = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    chunk = (B, l, S, H, d)
    t_max = sh["p_max"] + l
    caches = [ca2.Cache(B, H, d, S, l, sh["p_max"], sh["p_spatial"], sh["tpe_len"], "bf16") for _ in range(L)]
    first = [_randn((B, 1, S, H, d), gen, bf) for _ in range(4)]
    for c in caches:
        c.ca2_cache_write(*first)                    # the conditioning frame
    sets = [tuple(_randn(chunk, gen, bf) for _ in range(3)) for _ in range(L)]
    qc, kt, vt, ks, vs = (_randn(chunk, gen, bf) for _ in range(5))
    full = [tuple(_randn((B, t_max, S, H, d), gen, bf) for _ in range(3)) for _ in range(L)]
    out_t, out_s = torch.empty(chunk, dtype=bf, device="cuda"), torch.empty(chunk, dtype=bf, device="cuda")
    full_t = torch.empty((B, t_max, S, H, d), dtype=bf, device="cuda")
    full_s = torch.empty((B, t_max, S, H, d), dtype=bf, device="cuda")

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def denoise_cached():
        for _ in range(T_DENOISE):
            for li in range(L):
                q, k, v = sets[li]
                caches[li].ca2_denoise_attn(q, k, v, out_s, q, k, v, out_t)

    def write_all():
        for c in caches:
            c.ca2_denoise_attn(qc, ks, vs, out_s, qc, kt, vt, out_t, mode=ca2.CA2_SPATIAL_SELF)
            c.ca2_cache_write(kt, vt, ks, vs)

    steps = []
    frames = 1
    while frames < ROLLOUT_FRAMES:
        p_k = caches[0].ca2_cache_info_get()["p_k"]
        T = p_k + l

        def recompute():
            for _ in range(T_DENOISE):
                for li in range(L):
                    q, k, v = (x[:, :T] for x in full[li])
                    ca2.ca2_temporal_attn_frames(q, k, v, full_t[:, :T], causal=False)
                    ca2.ca2_spatial_attn_frames(q, k, v, full_s[:, :T])

        denoise_cached()                              # warm (reads the cache only)
        ms_den = timed(denoise_cached)
        ms_wr = timed(write_all)                      # advances every cache by one chunk
        recompute()
        ms_re = timed(recompute)
        # per denoising call and layer: only the cached path's temporal FLOPs grow with P_k
        flops = {"cached_spatial": spatial_flops(sh, l, sh["p_spatial"]),
                 "cached_temporal": temporal_flops(sh, l, p_k),
                 "recompute_spatial": spatial_flops(sh, T, 0),
                 "recompute_temporal": recompute_temporal_flops(sh, T)}
        # the same work at the spec rooflines (each kernel at max(bytes/HBM, flops/MFMA))
        def ideal_us(by, fl):
            return max(by / HBM_PEAK_GBS / 1e3, fl / MFMA_BF16_PEAK_TFLOPS / 1e6)
        calls = T_DENOISE * L
        ideal_c = calls * (ideal_us(spatial_bytes(sh, l, sh["p_spatial"]), flops["cached_spatial"]) +
                           ideal_us(temporal_bytes(sh, l, p_k), flops["cached_temporal"]))
        ideal_r = calls * (ideal_us(spatial_bytes(sh, T, 0), flops["recompute_spatial"]) +
                           ideal_us(recompute_bytes(sh, T), flops["recompute_temporal"]))
        steps.append(dict(p_k=p_k, frames_attended=T, cached_ms=round(ms_den + ms_wr, 3),
                          cached_write_pass_ms=round(ms_wr, 3), recompute_ms=round(ms_re, 3),
                          ideal_cached_denoise_ms=round(ideal_c / 1e3, 3),
                          ideal_recompute_ms=round(ideal_r / 1e3, 3),
                          flops_per_call_layer=flops))
        frames += l
    cum_c = cum_r = 0.0
    for st in steps:
        cum_c += st["cached_ms"]
        cum_r += st["recompute_ms"]
        st["cumulative_cached_ms"] = round(cum_c, 3)
        st["cumulative_recompute_ms"] = round(cum_r, 3)
    # the recompute kernels at the largest step, on their own rooflines
    T = t_max
    q, k, v = full[0]
    us_t = time_launches(lambda: ca2.ca2_temporal_attn_frames(q, k, v, full_t, causal=False), 50)
    us_s = time_launches(lambda: ca2.ca2_spatial_attn_frames(q, k, v, full_s), 20)
    by, fl_t, fl_s = recompute_bytes(sh, T), recompute_temporal_flops(sh, T), spatial_flops(sh, T, 0)
    for c in caches:
        c.close()
    ideal_c = sum(st["ideal_cached_denoise_ms"] for st in steps)
    ideal_r = sum(st["ideal_recompute_ms"] for st in steps)
    return {"workload": sh["name"], "layers": L, "denoise_calls_per_step": T_DENOISE,
            "steps": steps, "total_speedup": round(cum_r / cum_c, 3),
            "total_speedup_at_spec_rooflines": round(ideal_r / ideal_c, 3),
            "recompute_kernels_at_T%d" % T: {
                "temporal_bidirectional": {"us": round(us_t, 3), "bytes": by, "flops": fl_t,
                                           "achieved_gbs": round(by / us_t / 1e3, 1),
                                           "frac_hbm": round(by / us_t / 1e3 / HBM_PEAK_GBS, 4)},
                "spatial_self_frames": {"us": round(us_s, 3), "flops": fl_s,
                                        "achieved_tflops": round(fl_s / us_s / 1e6, 1),
                                        "frac_mfma": round(fl_s / us_s / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}}}


def measured_ceilings():
    """What the box sustains, beside the vendor figures: HBM from the
    library's own cache-write copy kernel moving a 1.21 GB working set (well
    past the 256 MB Infinity Cache: 64 batch entries x 8 frames of K and V,
    read and written), and dense bf16 MFMA from the vendor GEMM (torch.matmul,
    8192^3) -- the rate the matrix cores and the clock the part holds under
    full MFMA load actually give."""
    import torch
    from causal_kv_cache_amd import ca2
    B, H, d, S, l = 64, 16, 72, 256, 8
    c = ca2.Cache(B, H, d, S, l, 8, 0, 16, "bf16")
    kv = [torch.empty((B, l, S, H, d), dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(2)]
    moved = 2 * 2 * B * l * S * H * d * 2          # K and V, read and written
    us_copy = time_launches(lambda: c.ca2_cache_write(kv[0], kv[1], None, None), 10)
    c.close()
    del kv
    n = 8192
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    us_mm = time_launches(lambda: torch.matmul(a, b), 10)
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": round(moved / us_copy / 1e3, 1), "hbm_copy_bytes": moved,
            "mfma_bf16_gemm_tflops": round(2 * n ** 3 / us_mm / 1e6, 1),
            "how": "HBM: ca2_cache_write copying 64 x 8 frames of K and V (read + write bytes / time); "
                   "MFMA: torch.matmul bf16 8192^3 (vendor GEMM)"}


def kernel_mode(kernel, workload, reps):
    """Launch one kernel of one workload `reps` times (for profilers)."""
    import torch
    from causal_kv_cache_amd import ca2
    sh = WORKLOADS[workload]
    if kernel in ("qkv_proj", "qkv_proj_stage"):
        r = write_case(reps, rounds=1, only=kernel)[kernel]
        return {"kernel": kernel, "workload": workload, "reps": reps, "avg_us": r["us"], "flops": r["flops"]}
    # the same buffers and rotation as the benchmark's per-kernel table
    w = main_workload() if sh is AR_STEP else Workload(sh, 2, seed=99)
    if kernel == "cache_write":
        qc, kt, vt, ks, vs = w.clean
        fn = lambda: w.cache.ca2_cache_write(kt, vt, ks, vs)
    else:
        fn = launchers(w)[kernel]
    us = time_launches(fn, reps, rounds=1)      # exactly 1 + reps launches, all traced
    return {"kernel": kernel, "workload": workload, "reps": reps, "avg_us": round(us, 3)}


def cpu_baseline(budget_s: float):
    """The oracle, as it stands, on the same workload shape: whole denoising
    calls (temporal + prefix spatial attention, float64) until `budget_s`."""
    import numpy as np
    import synth
    from oracle import RolloutOracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:
        threads, blas = len(os.sched_getaffinity(0)), "?"
    sh = dict(synth.WORKLOADS["ar_step_s256"])
    o = RolloutOracle(sh, 1)
    for wsz in (1, 8, 8, 8):
        o.write(o.next_frames(wsz))
    calls = 0
    t0 = time.perf_counter()
    while True:
        o.denoise_outputs(4, 50 - calls % 50)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 50:
            break
    tokens = calls * sh["B"] * sh["l"] * sh["S"]
    return {"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} whole denoising calls (temporal + prefix spatial attention, float64 "
                      f"numpy, BLAS {blas}) at the 256-token shape with the queue full, "
                      f"{el:.1f} s; cache-writing pass not included",
            "seconds": el}


def cpu_rollout():
    """The oracle's 80-frame rollout (rollout_80f: B1, 256 tokens, 16 x 72,
    chunk 8, P_max 41, P' 3; 1 conditioning frame + 10 AR steps, each 50
    denoising calls and one cache-writing pass), float64 as it stands. A
    whole rollout is 500 denoising calls (~3 min on 16 cores), so the sample
    is one denoising call and one cache-writing pass at each distinct queue
    length the rollout passes through (P_k = 1, 9, 17, 25, 33, 41), each
    timed once in rollout order; the rollout time is their sum weighted by
    the number of AR steps at that P_k. Returns seconds and the sample."""
    import synth
    from oracle import RolloutOracle
    sh = dict(synth.WORKLOADS["rollout_80f"])
    l = sh["l"]
    o = RolloutOracle(sh, 2)
    o.write(o.next_frames(1))
    per_pk = {}
    steps_at = {}
    frames = 1
    while frames < 81:
        pk = o.queue.p_k
        steps_at[pk] = steps_at.get(pk, 0) + 1
        if pk not in per_pk:
            t0 = time.perf_counter()
            o.denoise_outputs(1 + frames // l, 0)
            t1 = time.perf_counter()
            o.write_pass_outputs(o.next_frames(l))
            t2 = time.perf_counter()
            per_pk[pk] = (t1 - t0, t2 - t1)
        o.write(o.next_frames(l))
        frames += l
    total = sum(n * (50 * per_pk[pk][0] + per_pk[pk][1]) for pk, n in steps_at.items())
    return {"seconds": round(total, 2),
            "per_p_k_s": {str(pk): [round(a, 4), round(b, 4)] for pk, (a, b) in per_pk.items()},
            "ar_steps_at_p_k": {str(k): v for k, v in steps_at.items()},
            "sample": "one denoising call (temporal + prefix spatial attention) and one cache-writing pass "
                      "(temporal + self spatial attention) per distinct P_k, float64; rollout = sum over AR "
                      "steps of 50 calls + 1 pass at that step's P_k"}


def cpu_per_kernel():
    """The oracle's temporal and prefix-spatial attention, as they stand
    (float64 numpy), timed per call on the host cores: whole calls at the
    256-token shape; at the batched 32x32-latent shape a stated sample of each
    call scaled to a whole call (rows, and (batch, frame, head) pairs, are
    independent, so the work scales linearly). Inputs are drawn before timing."""
    import numpy as np
    from oracle import temporal_attn_ref, spatial_attn_ref
    rng = np.random.default_rng(3)

    def draw(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    res = {}
    for sh, tb, sample in ((AR_STEP, AR_STEP["B"], None), (LARGE, 1, "spatial: 1 of 1024 (batch, frame, head)")):
        l, S, H, d, P, Ps = sh["l"], sh["S"], sh["H"], sh["d"], sh["p_max"], sh["p_spatial"]
        q, k, v = (draw(tb, l, S, H, d) for _ in range(3))
        rk, rv = draw(tb, P, S, H, d), draw(tb, P, S, H, d)
        t_t = timed(lambda: temporal_attn_ref(q, k, v, rk, rv, list(range(P)), d ** -0.5)) * sh["B"] / tb
        del rk, rv
        if sample:
            qs, ks_, vs_ = (x[:1, :1, :, :1] for x in (q, k, v))
            pk, pv = draw(1, Ps, S, 1, d), draw(1, Ps, S, 1, d)
            scale_up = sh["B"] * l * H
        else:
            qs, ks_, vs_ = q, k, v
            pk, pv = draw(sh["B"], Ps, S, H, d), draw(sh["B"], Ps, S, H, d)
            scale_up = 1
        t_s = timed(lambda: spatial_attn_ref(qs, ks_, vs_, pk, pv, list(range(Ps)), d ** -0.5, "prefix")) * scale_up
        res[sh["name"]] = {"temporal_s_per_call": round(t_t, 4), "spatial_prefix_s_per_call": round(t_s, 4),
                           "sample": ("whole calls" if not sample else
                                      f"temporal: batch entry 1 of {sh['B']}; {sample}; scaled to a whole call")}
    return res


TRAFFIC_KERNELS = {   # --kernel name -> (kernel-name substring, source file)
    "cache_write": ("copy_frames_kernel", "cache_write.hip"),
    "temporal": ("temporal_attn_ds_kernel", "temporal_attn.hip"),
    "spatial_prefix": ("spatial_attn_pipe_kernel", "spatial_attn.hip"),
    "spatial_self": ("spatial_attn_pipe_kernel", "spatial_attn.hip"),
    "denoise_fused": ("denoise_call_kernel", "spatial_attn.hip"),
    "qkv_proj": ("qkv_proj_kernel<false>", "qkv_proj.hip"),
    "qkv_proj_stage": ("qkv_proj_kernel<true>", "qkv_proj.hip"),
}


def algorithmic_bytes(kernel, workload):
    sh = WORKLOADS[workload]
    n, pk, ps = sh["l"], sh["p_max"], sh["p_spatial"]
    C = sh["H"] * sh["d"]
    if kernel == "cache_write":
        return write_bytes(sh, n)
    if kernel == "temporal":
        return temporal_bytes(sh, n, pk)
    if kernel == "spatial_prefix":
        return spatial_bytes(sh, n, ps)
    if kernel == "spatial_self":
        return spatial_bytes(sh, n, 0)
    if kernel == "denoise_fused":
        return spatial_bytes(sh, n, ps) + temporal_bytes(sh, n, pk)
    m = sh["B"] * n * sh["S"]
    x_w = 2 * (m * C + 3 * C * C)                      # X and W read once
    if kernel == "qkv_proj":
        return x_w + 2 * 3 * m * C                     # Q, K, V written
    # fused stage: Q out, K/V into the ring, the last P' frames' K/V into the
    # spatial buffer, the frames' TPE rows (fp32) read once
    return x_w + 2 * 3 * m * C + 2 * 2 * sh["B"] * min(n, ps) * sh["S"] * C + 4 * n * 3 * C


def traffic_summary(d, reps):
    """profiles/traffic.json from rocprofv3 counter runs of `bench.py --kernel
    K --workload W --reps R`: d/rd_K_W (TCC_EA0_RDREQ_sum, TCC_EA0_RDREQ_32B_sum,
    TCC_EA0_RDREQ_64B_sum) and d/wr_K_W (WRITE_SIZE). Read bytes follow the
    counters' definitions: RDREQ counts every L2-to-memory read request, of
    32, 64 or 128 bytes, and the 32- and 64-byte ones are counted apart, so
    bytes = 32 RDREQ_32B + 64 RDREQ_64B + 128 (RDREQ - RDREQ_32B - RDREQ_64B).
    (The stock FETCH_SIZE expression prices every request that is neither
    32-byte nor counted by TCC_BUBBLE at 64 bytes; on this part TCC_BUBBLE
    reads 0 while the requests are 128-byte, so FETCH_SIZE is half the bytes
    read -- the copy kernel's known 51,904,512 bytes confirm 128 per request.)
    Write bytes are WRITE_SIZE (64- and 32-byte write requests, priced as
    such). Means over the last `reps` dispatches of the kernel (the timed
    launches)."""
    import csv
    import collections

    def means(path, name):
        rows = list(csv.DictReader(open(os.path.join(path, "run_counter_collection.csv"))))
        by = collections.defaultdict(list)
        for r in rows:
            if name in r["Kernel_Name"]:
                by[r["Counter_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v[-reps:]) / len(v[-reps:]) for k, v in by.items()}, \
            next((r["Kernel_Name"] for r in rows if name in r["Kernel_Name"]), "")

    # entries of (kernel, workload) pairs not counted in this directory are
    # kept from the existing file (each carries the hash of the source it was
    # counted on, so a stale one is recognised and not reported)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    old = json.load(open(path))["kernels"] if os.path.exists(path) else {}
    out = {"method": traffic_summary.__doc__.split("\n\n")[0].replace("\n", " "), "kernels": dict(old)}
    for entry in sorted(os.listdir(d)):
        if not entry.startswith("rd_") or entry.endswith(".log"):
            continue
        tag = entry[3:]
        kernel = next(k for k in sorted(TRAFFIC_KERNELS, key=len, reverse=True) if tag.startswith(k + "_"))
        workload = tag[len(kernel) + 1:]
        name, src = TRAFFIC_KERNELS[kernel]
        rd, kname = means(os.path.join(d, entry), name)
        wr, _ = means(os.path.join(d, "wr_" + tag), name)
        r, r32, r64 = rd["TCC_EA0_RDREQ_sum"], rd["TCC_EA0_RDREQ_32B_sum"], rd["TCC_EA0_RDREQ_64B_sum"]
        read = 32 * r32 + 64 * r64 + 128 * (r - r32 - r64)
        write = wr["WRITE_SIZE"] * 1024
        alg = algorithmic_bytes(kernel, workload)
        out["kernels"][f"{kernel}@{workload}"] = {
            "kernel_name": kname, "rdreq": round(r), "rdreq_32b": round(r32), "rdreq_64b": round(r64),
            "read_bytes": round(read), "write_size_kib": round(wr["WRITE_SIZE"], 1),
            "hbm_bytes_per_launch": round(read + write), "algorithmic_bytes": alg,
            "ratio_to_algorithmic": round((read + write) / alg, 3),
            "source": src, "source_sha256_16": source_hash(kernel)}
    out["kernels"] = dict(sorted(out["kernels"].items()))
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~0.4 s of timed steps: long enough to average over clock and
    # box-to-box jitter, short against the rest of the run
    ap.add_argument("--steps", type=int, default=300)
    # untimed steps first: the clock ramps up over the first few ms of load,
    # and 3 warmup steps (~5 ms) left ~4 % of that ramp in the timed steps
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-large", action="store_true")
    ap.add_argument("--no-rollout", action="store_true")
    ap.add_argument("--kernel", choices=KERNELS, help="only launch this kernel (profiling mode)")
    ap.add_argument("--workload", choices=tuple(WORKLOADS), default=AR_STEP["name"])
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--traffic-summary", metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 counter runs in DIR (no GPU needed)")
    ap.add_argument("--spatial-variant", type=int, default=0,
                    help="profiling mode: force the bf16 spatial launch variant (0 = by size)")
    ap.add_argument("--temporal-variant", type=int, default=0,
                    help="profiling mode: force the bf16 temporal kernel (0 = default dimension-split, "
                         "2 = matrix-core rows)")
    args = ap.parse_args()
    if args.traffic_summary:
        print(json.dumps(traffic_summary(args.traffic_summary, args.reps), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from causal_kv_cache_amd import ca2
    ca2.load()
    torch.cuda.set_device(0)
    if args.kernel:
        ca2.ca2_set_spatial_variant(args.spatial_variant)
        ca2.ca2_set_temporal_variant(args.temporal_variant)
        print(json.dumps(kernel_mode(args.kernel, args.workload, args.reps)), flush=True)
        return

    w = main_workload()
    for _ in range(args.warmup):
        w.ar_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        w.ar_step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    tokens = args.steps * T_DENOISE * AR_STEP["B"] * AR_STEP["l"] * AR_STEP["S"]
    value = tokens / wall

    loop_eager, loop_two, loop_graph = denoise_loop_graph(w, 10)
    kt = kernel_table(w, args.kernel_reps, fused=True)
    # dominant kernel of the step: largest total time per step (the denoising
    # calls run as fused launches; the cache-writing pass runs the stand-alone
    # temporal and self-mode spatial kernels once each)
    per_step = {"denoise_fused": T_DENOISE * kt["denoise_fused"]["us"],
                "temporal_attn": kt["temporal_attn"]["us"],
                "spatial_attn_self": kt["spatial_attn_self"]["us"]}
    dom = max(per_step, key=per_step.get)
    d = kt[dom]
    kname = {"denoise_fused": "denoise_fused", "temporal_attn": "temporal",
             "spatial_attn_self": "spatial_self"}[dom]
    roofline = {"bound": d["bound"], "achieved": round(d["achieved"], 3), "peak": d["peak"],
                "unit": d["unit"], "frac": round(d["frac"], 4),
                "traffic": traffic_for(kname, AR_STEP["name"]),
                "kernel": dom,
                "per_launch": {"flops": d["flops"], "bytes": d["bytes"], "avg_us": round(d["us"], 3)}}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": AR_STEP["name"], "batch": 1, "heads": 16, "head_dim": 72, "tokens": 256,
                   "chunk": 8, "p_max": 25, "p_k": 25, "p_spatial": 3, "denoise_calls_per_step": T_DENOISE},
        "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "denoise_loop_50_calls_ms": {"eager": round(loop_eager, 4), "eager_two_launches_per_call": round(loop_two, 4),
                                     "hip_graph_replay": round(loop_graph, 4)},
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                    for k, r in kt.items()},
    }
    del w
    torch.cuda.empty_cache()
    ceil = measured_ceilings()
    for r in result["kernels"].values():
        meas = ceil["hbm_copy_gbs"] if r["bound"] == "hbm" else ceil["mfma_bf16_gemm_tflops"]
        r["frac_of_measured"] = round(r["achieved"] / meas, 4)
    result["measured_ceilings"] = ceil
    result["roofline"]["measured_peak"] = (ceil["hbm_copy_gbs"] if roofline["bound"] == "hbm"
                                           else ceil["mfma_bf16_gemm_tflops"])
    result["roofline"]["frac_of_measured"] = round(roofline["achieved"] / result["roofline"]["measured_peak"], 4)

    if not args.no_large:
        wl = Workload(LARGE, 2, seed=99)
        kl = kernel_table(wl, max(10, args.kernel_reps // 10))
        result["large"] = {"workload": LARGE["name"],
                           "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                                           for kk, vv in r.items()} for k, r in kl.items()},
                           "temporal_traffic": traffic_for("temporal", LARGE["name"]),
                           "spatial_traffic": traffic_for("spatial_prefix", LARGE["name"])}
        del wl
        torch.cuda.empty_cache()
        result["write_case"] = write_case(max(10, args.kernel_reps // 10))
        torch.cuda.empty_cache()
    if not args.no_rollout:
        result["rollout_cached_vs_recompute"] = rollout_compare()
        torch.cuda.empty_cache()

    if not args.no_cpu:
        cb = cpu_baseline(args.cpu_seconds)
        cb.pop("seconds", None)
        cb["value"] = round(cb["value"], 2)
        per = cpu_per_kernel()
        gpu = {AR_STEP["name"]: result.get("kernels", {}), LARGE["name"]: result.get("large", {}).get("kernels", {})}
        for wl, r in per.items():
            for name, key in (("temporal_attn", "gpu_temporal_us"), ("spatial_attn_prefix", "gpu_spatial_prefix_us")):
                if name in gpu.get(wl, {}):
                    r[key] = round(gpu[wl][name]["us"], 3)
        cb["per_kernel"] = per
        ro = cpu_rollout()
        gpu_ro = result.get("rollout_cached_vs_recompute")
        if gpu_ro:
            # the GPU figure for the same rollout: one attention layer's share of the timed 8-layer rollout
            ro["gpu_seconds_one_layer"] = round(gpu_ro["steps"][-1]["cumulative_cached_ms"] / 1e3 /
                                                gpu_ro["layers"], 4)
        cb["rollout_80f"] = ro
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
