"""QKV projection of the clean chunk (float64). Test infrastructure only.

The cache-writing stage of the Ca2-VDM notes (overall framework: each
autoregressive step ends with one forward pass of the denoised chunk that
computes and stores its K/V) needs the chunk's K and V; in a transformer block
these come from a linear projection of the chunk's tokens.
"""
from __future__ import annotations

import numpy as np


def qkv_proj_ref(x, w):
    """Y = X W^T split into Q, K, V.

    x: [M][C_in] tokens (rows are (b, frame, s) in the [B][n][S] order);
    w: [3*C][C_in], the row-major weight of a linear layer whose output
    columns are Q (0..C-1), K (C..2C-1), V (2C..3C-1).
    Returns three float64 [M][C] arrays.

    Pinned by one-hot inputs (each output row is a column of W^T, exactly),
    by a triple-loop brute force on tiny shapes, and by linearity.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    C3, Cin = w.shape
    assert x.shape[1] == Cin and C3 % 3 == 0
    C = C3 // 3
    y = x @ w.T
    return y[:, :C], y[:, C:2 * C], y[:, 2 * C:]
