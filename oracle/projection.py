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


def qkv_proj_tpe_ref(x, w, tpe_rows, first_frame, n_frames, tokens):
    """Y = X W^T + R[tpe(frame of the row)], split into Q, K, V.

    The cyclic temporal position embedding (Ca2-VDM notes, key design 4,
    Cyclic-TPEs) is bound into the cached K/V: the K/V of a clean frame are
    computed once, with the embedding of that frame's cyclic index, and keep
    it while they sit in the queue. Reading taken for where it enters (the
    pages do not say): the embedding vector e of index i is added to every
    token of the frame before the projection, so the projected output gains
    the row e W^T; ``tpe_rows`` holds those projected rows, one per index
    ([L_tpe][3*C]), and the row of frame F is tpe_rows[F mod L_tpe] with frame
    0 the conditioning frame.

    x: [M][C_in] with rows in [B][n][S] order (M = B * n_frames * tokens), the
    n frames being first_frame .. first_frame + n_frames - 1;
    w: [3*C][C_in]. Returns three float64 [M][C] arrays.

    Pinned by x = 0 (each row equals its frame's table row exactly, which
    recovers the index map) and by distributivity against projecting
    x + e[index] directly with a table built as e W^T.
    """
    from .cache import tpe_index_ref
    x = np.asarray(x, dtype=np.float64)
    tpe_rows = np.asarray(tpe_rows, dtype=np.float64)
    M = x.shape[0]
    assert M % (n_frames * tokens) == 0
    idx = tpe_index_ref(first_frame, n_frames, tpe_rows.shape[0])
    q, k, v = qkv_proj_ref(x, w)
    y = np.concatenate([q, k, v], 1)
    for r in range(M):
        y[r] += tpe_rows[idx[(r // tokens) % n_frames]]
    C = y.shape[1] // 3
    return y[:, :C], y[:, C:2 * C], y[:, 2 * C:]
