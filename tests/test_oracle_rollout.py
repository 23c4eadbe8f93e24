"""Oracle rollout on the tiny fp32 workload: queue states, TPE indices and
cached attention == brute-force recompute at every denoising call (CPU)."""
import numpy as np
import pytest

import synth
from oracle import RolloutOracle, full_recompute_temporal_ref, ar_schedule, spatial_attn_ref

TINY = synth.WORKLOADS["tiny_fp32"]


def _run(p0, seed=11):
    o = RolloutOracle(TINY, seed)
    l = TINY["l"]
    log = []
    for frames in ar_schedule(p0, l):
        o.write_pass_outputs(frames)
        o.write(frames)
    for ar in range(1, TINY["ar_steps"] + 2):        # + one denoise-only step after the last write
        frames = o.next_frames(l)
        tpe = o.tpe(l)
        for t in range(TINY["denoise_steps"], 0, -1):
            temporal, spatial = o.denoise_outputs(ar, t)
            # brute force over the whole sequence (clean frames + this chunk)
            q = o.noisy("q", ar, t, l)
            k = o.noisy("k", ar, t, l)
            v = o.noisy("v", ar, t, l)
            n0 = o.frames_written
            kseq = np.concatenate([o.clean("kt", range(n0)), k], 1)
            vseq = np.concatenate([o.clean("vt", range(n0)), v], 1)
            ref = full_recompute_temporal_ref(q, kseq, vseq, n0, TINY["p_max"], o.scale)
            assert np.max(np.abs(temporal - ref)) <= 1e-12
            # spatial prefix = last P' clean frames
            pf = list(range(max(0, n0 - TINY["p_spatial"]), n0))
            ks, vs = o.clean("ks", pf), o.clean("vs", pf)
            ref_s = spatial_attn_ref(q, k, v, ks, vs, list(range(len(pf))), o.scale, "prefix")
            assert np.max(np.abs(spatial - ref_s)) <= 1e-13
        log.append((tpe, o.queue.frame_ids(), o.queue.p_k))
        if ar <= TINY["ar_steps"]:
            o.write_pass_outputs(frames)
            o.write(frames)
    return log


def test_rollout_start_one_frame():
    log = _run(1)
    assert [p for _, _, p in log] == [1, 5, 9, 9]
    assert log[0][0] == [1, 2, 3, 4]
    assert log[2][0] == [9, 10, 11, 12]
    assert log[3][0] == [0, 1, 2, 3]                 # 13..16 wrap on a table of 13
    assert log[3][1] == list(range(4, 13))           # post-eviction queue


def test_rollout_start_full_queue():
    log = _run(9)
    assert [p for _, _, p in log] == [9, 9, 9, 9]
    assert log[0][1] == list(range(0, 9))
    assert log[1][1] == list(range(4, 13))
    assert log[1][0] == [0, 1, 2, 3]                 # second AR step wraps
    assert log[2][1] == list(range(8, 17))


def test_write_pass_self_mode_and_ring_bytes():
    o = RolloutOracle(TINY, 5)
    for frames in ar_schedule(9, TINY["l"]):
        o.write(frames)
    # ring holds frame-keyed K/V exactly at the queue's slots
    kt = o.clean("kt", o.queue.frame_ids())
    assert np.array_equal(o.ring_k[:, o.queue.slot_map()], kt)
    frames = o.next_frames(TINY["l"])
    temporal, spatial = o.write_pass_outputs(frames)
    # self mode ignores the spatial cache
    qc, ks, vs = o.clean("qc", frames), o.clean("ks", frames), o.clean("vs", frames)
    assert np.max(np.abs(spatial - spatial_attn_ref(qc, ks, vs, None, None, [], o.scale, "self"))) == 0
