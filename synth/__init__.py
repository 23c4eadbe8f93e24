"""Seeded synthetic inputs for the causal KV-cache attention workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds no attention, softmax, queue or position-index arithmetic:
only random draws, their rounding to the storage type, and counter-based keying.

Keying (counter-based): every tensor is drawn from its own Philox stream whose
key is the tuple ``(seed, tensor id, counter...)``. So any frame's data can be
regenerated on its own, and a cached path and a full-recompute path that ask for
the same frame see the same numbers.

* clean (cached) frames: ``frame_tensor(seed, "kt"|"vt"|"ks"|"vs", frame)`` -- one
  absolute frame id, all batch entries; the cache-writing pass produces exactly
  these K/V, so a frame's cached K/V never depends on later frames or on the
  denoising step.
* noisy chunk tensors: ``step_tensor(seed, "q"|"k"|"v", ar_step, t)`` -- redrawn
  per (autoregressive step, denoising step); ``t = 0`` is the cache-writing pass.

Values are i.i.d. N(0, std^2) drawn in float32. For bf16 storage they are then
rounded once to bfloat16 (round to nearest even); both the oracle (which upcasts
to float64) and the device (which receives the bf16 bit patterns) see those same
rounded values.
"""
from __future__ import annotations

import numpy as np

# Stable ids for the Philox key; never renumber (stored fixtures depend on them).
TENSOR_IDS = {
    "q": 1, "k": 2, "v": 3,          # noisy chunk, per (ar_step, t)
    "kt": 4, "vt": 5,                # temporal-layer K/V of a clean frame
    "ks": 6, "vs": 7,                # spatial-layer K/V of a clean frame
    "x": 8, "w": 9,                  # projection input / weight
    "qc": 10,                        # cache-writing-pass queries of a clean frame
}

DTYPES = ("f32", "bf16")


def _stream(seed: int, tensor: str, *counter: int) -> np.random.Generator:
    words = [int(seed), TENSOR_IDS[tensor]] + [int(c) for c in counter]
    if any(w < 0 for w in words):
        raise ValueError("seed and counters must be non-negative")
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(words)))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16. Inputs
    are finite normals here; NaN/Inf handling is not needed and not provided.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16-exact."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("values are not bfloat16-exact; call round_to_bf16 first")
    return (b >> np.uint32(16)).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array holding the values as stored in ``dtype`` ("f32" or "bf16")."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(seed: int, tensor: str, counter: tuple, shape, dtype: str = "f32",
           std: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, std^2) draws keyed by (seed, tensor, *counter), stored as ``dtype``."""
    g = _stream(seed, tensor, *counter)
    x = g.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return to_storage(x, dtype)


def frame_tensor(seed: int, tensor: str, frame: int, B: int, S: int, H: int, d: int,
                 dtype: str = "f32") -> np.ndarray:
    """[B][S][H][d] data of one clean frame with absolute id ``frame``."""
    return normal(seed, tensor, (0, frame, B, S, H, d), (B, S, H, d), dtype)


def frames_tensor(seed: int, tensor: str, frames, B: int, S: int, H: int, d: int,
                  dtype: str = "f32") -> np.ndarray:
    """[B][len(frames)][S][H][d]: the clean frames listed, in that order."""
    frames = list(frames)
    out = np.empty((B, len(frames), S, H, d), dtype=np.float32)
    for i, f in enumerate(frames):
        out[:, i] = frame_tensor(seed, tensor, f, B, S, H, d, dtype)
    return out


def step_tensor(seed: int, tensor: str, ar_step: int, t: int, B: int, n: int, S: int,
                H: int, d: int, dtype: str = "f32") -> np.ndarray:
    """[B][n][S][H][d] noisy-chunk data for one (autoregressive step, denoising step)."""
    return normal(seed, tensor, (1, ar_step, t, B, n, S, H, d), (B, n, S, H, d), dtype)


def weight(seed: int, rows: int, cols: int, std: float, dtype: str = "bf16") -> np.ndarray:
    """[rows][cols] N(0, std^2) weight matrix."""
    return normal(seed, "w", (2, rows, cols), (rows, cols), dtype, std=std)


def activations(seed: int, rows: int, cols: int, dtype: str = "bf16") -> np.ndarray:
    """[rows][cols] N(0, 1) activation matrix (projection input)."""
    return normal(seed, "x", (3, rows, cols), (rows, cols), dtype)


# ---------------------------------------------------------------------------
# Workload shapes. Each entry names what the workload is and its sizes.
# ---------------------------------------------------------------------------
WORKLOADS = {
    # tiny fp32 parity case: 3 AR steps x 2 denoising steps
    "tiny_fp32": dict(B=1, H=2, d=16, S=16, l=4, p_max=9, p_spatial=1, tpe_len=13,
                      dtype="f32", ar_steps=3, denoise_steps=2),
    # one AR step at the 256x256 latent shape, queue full at P_max = 25
    "ar_step_s256": dict(B=1, H=16, d=72, S=256, l=8, p_max=25, p_spatial=3, tpe_len=33,
                         dtype="bf16", ar_steps=1, denoise_steps=50),
    # 80-frame rollout from one clean frame, P_max = 41, TPE table 49
    "rollout_80f": dict(B=1, H=16, d=72, S=256, l=8, p_max=41, p_spatial=3, tpe_len=49,
                        dtype="bf16", ar_steps=10, denoise_steps=50),
    # batched 32x32 latent, spatial-heavy
    "large_b8_s1024": dict(B=8, H=16, d=72, S=1024, l=8, p_max=25, p_spatial=3, tpe_len=33,
                           dtype="bf16", ar_steps=1, denoise_steps=1),
    # cache write + projection + memory contrast
    "write_b4": dict(B=4, H=16, d=72, S=256, l=8, p_max=41, p_spatial=3, tpe_len=49,
                     dtype="bf16", ar_steps=1, denoise_steps=50),
}
