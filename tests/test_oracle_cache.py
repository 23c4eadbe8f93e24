"""Oracle queue / spatial cache / TPE bookkeeping pinned by brute force and
invariants; bytes formula checked against the pages' memory table (CPU)."""
import json
import os

import numpy as np
import pytest

from oracle import TemporalQueue, SpatialCache, tpe_index_ref, bytes_resident_ref
from oracle.rollout import ar_schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_force_ring(p_max, writes):
    """A physical array of P_max slots: each new frame overwrites the slot
    holding the oldest frame, or the lowest empty slot. Returns (queued ids in
    age order, their slots)."""
    slots = [None] * p_max
    frame = 0
    for w in writes:
        for _ in range(w):
            if None in slots:
                s = slots.index(None)
            else:
                s = min(range(p_max), key=lambda i: slots[i])
            slots[s] = frame
            frame += 1
    held = sorted(f for f in slots if f is not None)
    return held, [slots.index(f) for f in held]


@pytest.mark.parametrize("p_max,writes", [
    (9, [1, 4, 4, 4, 4, 4, 4]),
    (41, [1] + [8] * 12),
    (25, [1, 8, 8, 8, 8]),
    (5, [1, 2, 3, 7, 1, 1, 9]),       # writes larger than P_max evict within the write
    (1, [1, 1, 3]),
])
def test_queue_matches_brute_force(p_max, writes):
    q = TemporalQueue(p_max)
    total = 0
    for w in writes:
        q.write(range(total, total + w))
        total += w
        ids, slots = _brute_force_ring(p_max, [total])
        assert q.frame_ids() == ids == list(range(max(0, total - p_max), total))
        assert q.slot_map() == slots


def test_queue_tiny_schedules():
    # P0 = 1: 1 -> 5 -> 9, first eviction on the third AR step's write
    q = TemporalQueue(9)
    sizes = []
    for w in [1, 4, 4, 4]:
        q.write(range(sum(sizes), sum(sizes) + w))
        sizes.append(w)
    assert q.frame_ids() == list(range(4, 13))
    assert q.slot_map() == [4, 5, 6, 7, 8, 0, 1, 2, 3]


def test_spatial_cache_logical_frames():
    c = SpatialCache(3)
    c.write([0])
    assert c.logical_frames() == [0, 0, 0]
    c.write(range(1, 9))
    assert c.logical_frames() == [6, 7, 8]
    c.write([9])
    assert c.logical_frames() == [7, 8, 9]
    c1 = SpatialCache(1)
    c1.write([0]); assert c1.logical_frames() == [0]
    c1.write(range(1, 5)); assert c1.logical_frames() == [4]
    c0 = SpatialCache(0)
    c0.write(range(3)); assert c0.logical_frames() == []


def test_spatial_cache_slots_hold_logical_frames():
    c = SpatialCache(3)
    rng = np.random.default_rng(0)
    total = 0
    for _ in range(20):
        w = int(rng.integers(1, 9))
        c.write(range(total, total + w))
        total += w
        frames = c.logical_frames()
        assert frames == [max(0, total - 3 + j) for j in range(3)]
        assert [c.slots[s] for s in c.slot_map()] == frames


def test_tpe_walk_equals_modulo_and_wraps():
    for L in (13, 33, 49):
        for first in range(0, 3 * L):
            assert tpe_index_ref(first, 8, L) == [(first + i) % L for i in range(8)]
    # 80-frame rollout, table of 49: frames 49..56 wrap to 0..7
    assert tpe_index_ref(49, 8, 49) == list(range(8))
    # tiny case started full (9 frames): second AR step's frames 13..16 -> 0..3
    assert tpe_index_ref(13, 4, 13) == [0, 1, 2, 3]


@pytest.mark.parametrize("p_max,l,L", [(9, 4, 13), (41, 8, 49), (25, 8, 33)])
def test_tpe_distinct_in_every_window(p_max, l, L):
    idx = tpe_index_ref(0, 400, L)
    w = p_max + l
    for s in range(0, 400 - w):
        assert len(set(idx[s:s + w])) == w


def test_ar_schedule():
    assert ar_schedule(1, 4) == [[0]]
    assert ar_schedule(9, 4) == [[0], [1, 2, 3, 4], [5, 6, 7, 8]]
    assert ar_schedule(25, 8)[-1] == list(range(17, 25))
    with pytest.raises(ValueError):
        ar_schedule(8, 4)


def test_bytes_resident_reproduces_memory_table():
    with open(os.path.join(GOLDEN, "memory_table.json")) as f:
        g = json.load(f)
    a = g["assumptions"]
    for row in g["rows"]:
        b = bytes_resident_ref(1, a["tokens"], a["heads"], a["head_dim"], a["p_max"],
                               row["p_spatial"], a["elem_bytes"], depth=a["depth"])
        assert b == row["bytes"]
        assert round(b / 2 ** 30, 2) == row["kv_cache_gb"]


def test_bytes_resident_write_case():
    # B=4, 256 tokens, 16x72, P_max 41, P' 3, bf16: one shared cache vs T=50 copies
    b = bytes_resident_ref(4, 256, 16, 72, 41, 3, 2)
    assert b == 193_462_272 + 14_155_776 == 207_618_048
    assert 50 * b == 10_380_902_400


def _brute_force_ring_slots(p_max, nslots, total):
    """A physical array of nslots >= P_max slots written frame by frame: each
    new frame takes the lowest empty slot, else overwrites the slot holding
    the oldest frame physically present. The queue is the newest P_max of the
    frames present. Returns (queued ids in age order, their slots)."""
    slots = [None] * nslots
    for frame in range(total):
        if None in slots:
            s = slots.index(None)
        else:
            s = min(range(nslots), key=lambda i: slots[i])
        slots[s] = frame
    held = sorted(f for f in slots if f is not None)[-p_max:]
    return held, [slots.index(f) for f in held]


@pytest.mark.parametrize("p_max,l,writes", [
    (9, 4, [1, 4, 4, 4, 4, 4, 4]),
    (41, 8, [1] + [8] * 12),
    (25, 8, [1, 8, 8, 8, 8, 3, 8]),
    (1, 2, [1, 2, 1, 2, 2]),
])
def test_queue_with_staging_slots(p_max, l, writes):
    """P_max + l physical slots: placement equals the brute-force ring, and the
    slots a write fills held no queued frame before the write, so the new
    frames can be stored before the queue moves on."""
    q = TemporalQueue(p_max, slots=p_max + l)
    total = 0
    for w in writes:
        before = set(q.slot_map())
        landed = q.write(range(total, total + w))
        total += w
        assert not before & set(landed)
        assert len(set(landed)) == len(landed)
        ids, slots = _brute_force_ring_slots(p_max, p_max + l, total)
        assert q.frame_ids() == ids == list(range(max(0, total - p_max), total))
        assert q.slot_map() == slots


def test_queue_without_staging_slots_overwrites_queued_frames():
    """With exactly P_max slots a full queue's write lands on frames it still
    holds before the write (why a staged write needs the extra slots)."""
    q = TemporalQueue(5)
    q.write(range(5))
    before = set(q.slot_map())
    assert before & set(q.write(range(5, 7)))


def test_staging_slots_property():
    """Random P_max, chunk length and write sequences (each write 1..l frames):
    with P_max + l physical slots every write lands in slots that held no
    queued frame, and placement always equals the brute-force ring."""
    import hypothesis
    import hypothesis.strategies as st

    @hypothesis.settings(max_examples=120, deadline=None, derandomize=True)
    @hypothesis.given(p_max=st.integers(1, 12), l=st.integers(1, 6), data=st.data())
    def check(p_max, l, data):
        writes = data.draw(st.lists(st.integers(1, l), min_size=1, max_size=12))
        q = TemporalQueue(p_max, slots=p_max + l)
        total = 0
        for w in writes:
            before = set(q.slot_map())
            landed = q.write(range(total, total + w))
            total += w
            assert not before & set(landed)
            ids, slots = _brute_force_ring_slots(p_max, p_max + l, total)
            assert q.frame_ids() == ids and q.slot_map() == slots

    check()
