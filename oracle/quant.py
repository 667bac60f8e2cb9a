"""Weight-quantized rows combined with activation sparsity, in fp64.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .teal import magnitude_mask


def quantize_rows_int8(W):
    """Symmetric per-row int8 quantization: ``s_i = max_j |W_ij| / 127`` and
    ``q_ij = clip(round_half_even(W_ij / s_i), -127, 127)``; an all-zero row gets
    s_i = 0 and q = 0.  Returns (q int8 [K, N], s float64 [K]).

    Attribution notes, discussion: activation sparsity is compatible with weight
    quantization (W8A8, INT4) and the two savings combine.  Reading taken: weights
    only (activations stay in their own dtype), one scale per input row, so a
    skipped row skips its scale too."""
    W = np.asarray(W, dtype=np.float64)
    amax = np.abs(W).max(axis=1)
    s = amax / 127.0
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(W / safe[:, None]), -127, 127)
    q[s == 0] = 0
    return q.astype(np.int8), s


def masked_gemv_rows_int8(x, Wq, row_scale, t):
    """``y = sum over i with |x_i| > t of x_i * row_scale_i * Wq[i, :]`` (one token,
    the mask on x itself, the row scale applied to the kept rows only)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    q = np.asarray(Wq, dtype=np.float64)
    s = np.asarray(row_scale, dtype=np.float64)
    keep = magnitude_mask(x, t)
    idx = np.flatnonzero(keep)
    return (x[idx] * s[idx]) @ q[idx]
