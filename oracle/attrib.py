"""Attribution-based selection (external scores) in fp64.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from .topk import value_topk


def corrected_gxo(x, grad):
    """Corrected Gradient x Output score of every neuron of a layer, row by row:
    ``score_i = grad_i * x_i + 1/2 * |x_i| * sqrt(sum_k grad_k^2)``.

    Attribution notes, correction term: the first term is plain GxO, the second
    corrects the inter-layer dependency with the neuron's output magnitude times
    the L2 norm of the layer's gradient, scaled by 1/2.  ``x``, ``grad``:
    ``[n]`` or ``[rows, n]`` (one layer per row)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = np.atleast_2d(np.asarray(grad, dtype=np.float64))
    norm = np.sqrt((g * g).sum(axis=1, keepdims=True))
    return g * x + 0.5 * np.abs(x) * norm


def fraction_count(n: int, num: int, den: int) -> int:
    """Neurons kept at activation ratio num/den: ``ceil(num * n / den)``, exact."""
    return int(math.ceil(Fraction(num, den) * n))


def top_fraction(score, num: int, den: int):
    """Approach 1 of the attribution notes (implementation section): per layer,
    keep the top fraction of neurons by score (a fixed activation ratio per layer,
    not one threshold shared across layers).  Reading taken: the ratio num/den is
    exact, k = ceil(ratio * n), and the k largest scores are kept (by value: a
    negative attribution is the least important; ties to the smaller index).
    ``score``: ``[rows, n]``.  Returns a bool keep mask ``[rows, n]``."""
    s = np.atleast_2d(np.asarray(score, dtype=np.float64))
    rows, n = s.shape
    k = fraction_count(n, num, den)
    keep = np.zeros((rows, n), dtype=bool)
    for r in range(rows):
        keep[r, value_topk(s[r], k)] = True
    return keep


def head_masked_gemv(x, W, heads, head_dim: int):
    """Attention output projection restricted to the kept heads:
    ``y = sum over kept heads h of x[h*hd:(h+1)*hd] @ W[h*hd:(h+1)*hd, :]``.

    Attribution notes, implementation: in attention the neuron is a head (the
    SDPA output), and deactivating it zeroes the weights it connects to, here
    the head_dim-row block of the output projection.  ``W`` input-major
    ``[n_heads * head_dim, N]``; ``heads``: kept head indices."""
    x = np.asarray(x, dtype=np.float64).ravel()
    W = np.asarray(W, dtype=np.float64)
    y = np.zeros(W.shape[1])
    for h in np.asarray(heads, dtype=np.int64):
        sl = slice(int(h) * head_dim, (int(h) + 1) * head_dim)
        y += x[sl] @ W[sl]
    return y
