"""Autoregressive rollout driver over the oracle pieces. Test infrastructure only.

Ca2-VDM notes, overall framework (inference): each autoregressive step is a
denoising stage -- T model calls at different timesteps t, all reading the
cache -- followed by a cache-writing stage -- one pass of the denoised chunk at
t = 0 that computes and stores its K/V. Key design 4 bounds the temporal queue
at P_max frames; key design 5 keeps one chunk's worth of spatial K/V.

Synthetic stand-in for the model (see ``synth``): a clean frame's temporal and
spatial K/V are fixed per absolute frame id (the cache-writing pass yields
exactly those), and the noisy chunk's Q/K/V are redrawn per (AR step, t).
"""
from __future__ import annotations

import numpy as np

import synth
from .attention import temporal_attn_ref, spatial_attn_ref
from .cache import TemporalQueue, SpatialCache, tpe_index_ref


def ar_schedule(p0: int, l: int):
    """Chunks in which the first ``p0`` clean frames are written: the
    conditioning frame alone, then whole chunks of length l (the pages'
    prefix lengths are 1 + multiples of l -- training strategy section).
    Returns a list of frame-id lists."""
    if p0 < 1 or (p0 - 1) % l:
        raise ValueError("p0 must be 1 + a multiple of the chunk length")
    chunks = [[0]]
    f = 1
    while f < p0:
        chunks.append(list(range(f, f + l)))
        f += l
    return chunks


class RolloutOracle:
    """Cache state plus on-demand reference outputs for a rollout.

    ``shape``: dict with B, H, d, S, l, p_max, p_spatial, tpe_len, dtype.
    The ring is held as a float32 array at the queue's physical slots, so it
    is also the reference for the bytes the cache write must produce.
    """

    def __init__(self, shape: dict, seed: int):
        self.sh = dict(shape)
        self.seed = seed
        sh = self.sh
        self.queue = TemporalQueue(sh["p_max"])
        self.spatial = SpatialCache(sh["p_spatial"])
        self.frames_written = 0
        dims = (sh["B"], sh["p_max"], sh["S"], sh["H"], sh["d"])
        self.ring_k = np.zeros(dims, dtype=np.float32)
        self.ring_v = np.zeros(dims, dtype=np.float32)
        self.scale = 1.0 / np.sqrt(sh["d"])

    # -- synthetic data -------------------------------------------------
    def _dims(self):
        sh = self.sh
        return sh["B"], sh["S"], sh["H"], sh["d"]

    def clean(self, tensor: str, frames):
        B, S, H, d = self._dims()
        return synth.frames_tensor(self.seed, tensor, frames, B, S, H, d, self.sh["dtype"])

    def noisy(self, tensor: str, ar_step: int, t: int, n: int):
        B, S, H, d = self._dims()
        return synth.step_tensor(self.seed, tensor, ar_step, t, B, n, S, H, d, self.sh["dtype"])

    def spatial_prefix(self):
        """(ks, vs, slot_map) of the spatial cache in logical order, as
        [B][P'][S][H][d] arrays indexed by logical position."""
        frames = self.spatial.logical_frames()
        ks = self.clean("ks", frames)
        vs = self.clean("vs", frames)
        return ks, vs, list(range(len(frames)))

    # -- reference outputs ------------------------------------------------
    def temporal(self, q, k_new, v_new):
        return temporal_attn_ref(q, k_new, v_new, self.ring_k, self.ring_v,
                                 self.queue.slot_map(), self.scale)

    def spatial_out(self, q, k, v, mode):
        if mode == "prefix" and self.sh["p_spatial"] > 0:
            ks, vs, slots = self.spatial_prefix()
            if not slots:
                raise RuntimeError("prefix mode needs at least one clean frame")
            return spatial_attn_ref(q, k, v, ks, vs, slots, self.scale, "prefix")
        return spatial_attn_ref(q, k, v, None, None, [], self.scale, "self")

    def next_frames(self, n: int):
        return list(range(self.frames_written, self.frames_written + n))

    def tpe(self, n: int):
        return tpe_index_ref(self.frames_written, n, self.sh["tpe_len"])

    def write_pass_outputs(self, frames):
        """Cache-writing pass of clean ``frames`` (t = 0), before the write:
        temporal attention over the queue + the chunk, spatial self mode."""
        qc = self.clean("qc", frames)
        kt, vt = self.clean("kt", frames), self.clean("vt", frames)
        ks, vs = self.clean("ks", frames), self.clean("vs", frames)
        return self.temporal(qc, kt, vt), self.spatial_out(qc, ks, vs, "self")

    def write(self, frames):
        """Append ``frames`` to the queue (evicting past P_max) and refresh
        the spatial cache; the ring array receives the frames' K/V at the
        slots the queue assigns."""
        frames = list(frames)
        assert frames == self.next_frames(len(frames))
        slots = self.queue.write(frames)
        kt, vt = self.clean("kt", frames), self.clean("vt", frames)
        # only frames still queued survive; later writes to a slot win
        for i, (f, s) in enumerate(zip(frames, slots)):
            self.ring_k[:, s] = kt[:, i]
            self.ring_v[:, s] = vt[:, i]
        self.spatial.write(frames)
        self.frames_written += len(frames)
        return slots

    def denoise_outputs(self, ar_step: int, t: int):
        """(temporal, spatial-prefix) outputs of one denoising call."""
        n = self.sh["l"]
        q, k, v = (self.noisy(x, ar_step, t, n) for x in ("q", "k", "v"))
        return self.temporal(q, k, v), self.spatial_out(q, k, v, "prefix")
