"""Queue, spatial cache and cyclic position indices (integer bookkeeping).

Test infrastructure only; see oracle/__init__.py.
"""
from __future__ import annotations

from collections import deque
import itertools


class TemporalQueue:
    """FIFO queue of clean-frame ids with a fixed number of physical slots.

    Ca2-VDM notes, key design 4 (temporal KV-cache queue): the number of
    cached conditioning frames P_k grows by one chunk per autoregressive step;
    once it reaches P_max the oldest entries leave the queue, so its length
    stays P_max.

    Physical placement over ``slots`` physical slots (P_max unless more are
    asked for): a new frame goes to slot (head + length) mod slots, i.e.
    right after the newest entry; when the queue then holds more than P_max
    ids the oldest is dropped and ``head`` advances by one. The slot of
    logical position j is (head + j) mod slots. With slots >= P_max + n, the
    n frames of a write land in slots that held no queued frame before it, so
    they can be filled before the queue moves on.

    Pinned by brute force (a plain list that keeps the last P_max ids), by
    the invariant "queue == last min(N, P_max) frame ids" and, for the
    placement, by a last-writer-wins table of which frame each slot holds.
    """

    def __init__(self, p_max: int, slots: int | None = None):
        if p_max < 1:
            raise ValueError("p_max must be >= 1")
        self.p_max = p_max
        self.slots = p_max if slots is None else int(slots)
        if self.slots < p_max:
            raise ValueError("slots must be >= p_max")
        self.ids = deque()
        self.head = 0

    @property
    def p_k(self) -> int:
        return len(self.ids)

    def write(self, frame_ids):
        """Append frames (in order) and evict down to P_max. Returns the
        physical slot each written frame landed in."""
        slots = []
        for f in frame_ids:
            slot = (self.head + len(self.ids)) % self.slots
            self.ids.append(int(f))
            slots.append(slot)
            while len(self.ids) > self.p_max:
                self.ids.popleft()
                self.head = (self.head + 1) % self.slots
        return slots

    def frame_ids(self):
        return list(self.ids)

    def slot_map(self):
        """Physical slot of each logical position, oldest first."""
        return [(self.head + j) % self.slots for j in range(len(self.ids))]


class SpatialCache:
    """The spatial KV-cache: the last P' clean frames, by absolute id.

    Ca2-VDM notes, key design 5 (spatial KV-cache): since P' < l only the most
    recent chunk is needed; it is overwritten each autoregressive step and has
    no queue. Key design 3 uses the last P' prefix frames.

    Physical placement here: P' slots; each new frame that must be kept takes
    an empty slot if one exists (lowest index first), else the slot of the
    oldest frame held. Logical order is oldest to newest. While fewer than P'
    clean frames exist, the logical list is left-padded by repeating the oldest
    frame held (a reading: the pages are silent on this case; it keeps the
    (P'+1)S keys of key design 3, modelled on its self-repeat alignment).

    Pinned by hand-written logical lists per write sequence and, for the
    padding, by the closed form that attention over a prefix repeating a
    frame m times equals attention over the distinct frames with that frame's
    exponentials counted m times (hand-written multiplicities, loop-evaluated
    weighted softmax); padding with the newest frame, with the target frame,
    with zeros, or not at all each fails it.
    """

    def __init__(self, p_spatial: int):
        if p_spatial < 0:
            raise ValueError("p_spatial must be >= 0")
        self.p = p_spatial
        self.slots = [None] * p_spatial   # frame id held in each physical slot

    def write(self, frame_ids):
        keep = list(frame_ids)[-self.p:] if self.p else []
        for f in keep:
            if None in self.slots:
                s = self.slots.index(None)
            else:
                s = min(range(self.p), key=lambda i: self.slots[i])
            self.slots[s] = int(f)

    def held(self):
        return sorted(f for f in self.slots if f is not None)

    def logical_frames(self):
        held = self.held()
        if not held:
            return []
        return [held[0]] * (self.p - len(held)) + held

    def slot_map(self):
        return [self.slots.index(f) for f in self.logical_frames()]


def tpe_index_ref(first_frame: int, n: int, tpe_len: int):
    """Cyclic temporal-position-embedding indices of frames first_frame ..
    first_frame+n-1.

    Ca2-VDM notes, key design 4 (Cyclic-TPEs): once the generated length
    passes the length of the position table, new targets take indices that
    start again from the beginning while cached K/V keep the indices they were
    computed with. Reading: frame 0 is the conditioning frame and indices are
    taken in a cycle over the table, so index(frame) = frame mod L_tpe.

    Written as a walk around the table (no modulo) so the modulo formula in the
    library is checked against a different construction.
    """
    if tpe_len < 1 or n < 0 or first_frame < 0:
        raise ValueError("bad arguments")
    if first_frame > 10 ** 7:
        raise ValueError("walk limited to first_frame <= 1e7")
    cyc = itertools.cycle(range(tpe_len))
    return list(itertools.islice(cyc, first_frame, first_frame + n))


def bytes_resident_ref(B, S, H, d, p_max, p_spatial, elem_bytes, depth=1):
    """Bytes of one shared cache: temporal ring (P_max frames of K and V) plus
    the spatial buffer (P' frames of K and V), per layer times ``depth``.

    Ca2-VDM notes, key design 2 (cache sharing: storage does not depend on the
    number of denoising steps T) and the GPU-memory table (KV-cache GB at 50
    denoising steps, with and without prefix enhancement).
    """
    C = H * d
    per_layer = 2 * B * (p_max + p_spatial) * S * C * elem_bytes
    return per_layer * depth
