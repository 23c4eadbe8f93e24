"""Helpers for GPU tests: moving synth/oracle arrays to and from the device
and the numeric bars the GPU path is held to."""
import numpy as np
import torch

import synth

# fp32: |g - o| <= 1e-5 |o| + 1e-6 element-wise; bf16: max-abs <= 2e-2, and
# (a regression guard below that bar) the mean absolute error within 1 % of
# the mean output magnitude: rounding the inputs' products and P to bf16 and
# the output to bf16 costs a few tenths of a percent, so a systematic error
# of the size the max-abs bar still lets through shows up here.
F32_RTOL, F32_ATOL = 1e-5, 1e-6
BF16_ATOL = 2e-2
BF16_MEAN_REL = 1e-2


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array (bf16-exact for bf16) -> contiguous cuda tensor."""
    if dtype == "bf16":
        bits = synth.bf16_bits(x).view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    """cuda tensor -> float64 numpy array of its exact values."""
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def bits_to_f32(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns (from debug_copy) -> float32 values."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def empty_like_dev(shape, dtype: str) -> torch.Tensor:
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.empty(shape, dtype=td, device="cuda")


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        bound = F32_RTOL * np.abs(ref) + F32_ATOL
        worst = float(np.max(err - bound))
        assert worst <= 0, f"{what}: fp32 error exceeds 1e-5|o|+1e-6 by {worst:.3g} (max err {err.max():.3g})"
    else:
        m = float(err.max())
        assert m <= BF16_ATOL, f"{what}: bf16 max-abs error {m:.4g} > {BF16_ATOL}"
        mean_err, mean_ref = float(err.mean()), float(np.abs(ref).mean())
        assert mean_err <= BF16_MEAN_REL * mean_ref + 1e-5, \
            f"{what}: bf16 mean-abs error {mean_err:.3g} > 1% of mean |o| {mean_ref:.3g}"
    return float(err.max())
