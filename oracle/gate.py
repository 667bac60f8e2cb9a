"""Gate-score activation sparsity (CATS; intra-expert sparsity) in fp64.

Test infrastructure only (see the package docstring).

The gate projection runs densely and scores every neuron; only the neurons whose
gate activation survives a magnitude threshold (or the top-k of them) take part in
the up and down projections.
"""
from __future__ import annotations

import numpy as np

from .teal import calibrate_threshold, magnitude_mask, silu
from .topk import value_topk


def gate_activation(x, Wg):
    """``a = silu(x Wg^T)`` for every neuron: the gate activation that scores it.

    Wg neuron-major ``[d_ff, d_model]`` (row j = neuron j's gate weights); ``x`` is
    ``[d_model]`` or ``[M, d_model]``.  Returns ``(g, a)``.

    Intra-expert summary, system implementation: the gate projection is executed
    densely (a batched matrix product) to determine the activation scores.  TEAL
    slides, slides 5-6 (CATS): the score is the magnitude of SiLU(x W_gate).
    """
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(Wg, dtype=np.float64).T
    return g, silu(g)


def gate_score_mlp(x, Wg, Wu, Wd, t=None, k=None):
    """SwiGLU MLP in which the gate activation decides which neurons run.

    Intra-expert summary, system implementation: (1) dense gate projection,
    (2) threshold masking of the activation scores in a single O(n) pass (no
    top-k sort), (3) the up and down projections use only the active neurons'
    weights, gathered and packed densely before a dense matrix-vector product.
    TEAL slides, slides 5-6 (CATS): threshold |SiLU(x W_gate)|; W_up and W_down
    are pruned, the gate is not.

    Keep rule per token: ``|a_j| > t`` (strict, t compared as fp32 like every
    threshold of this package), or with ``k`` the k largest |a_j| (ties to the
    smaller neuron index).  Then for kept j: ``u_j = x . Wu[j]``,
    ``h_j = a_j u_j``; dropped neurons contribute nothing; ``y = sum_j h_j Wd[j]``.
    All three matrices neuron-major ``[d_ff, d_model]``.

    Returns a dict with g, a, keep (bool [M, d_ff]), h ([M, d_ff], 0 where dropped)
    and y ([M, d_model]); a 1-D ``x`` is treated as one token.
    """
    if (t is None) == (k is None):
        raise ValueError("exactly one of t (threshold) and k (top-k) is given")
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    Wu = np.asarray(Wu, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    g, a = gate_activation(x, Wg)
    M, n = a.shape
    if t is not None:
        keep = magnitude_mask(a, t)
    else:
        keep = np.zeros((M, n), dtype=bool)
        for m in range(M):
            keep[m, value_topk(np.abs(a[m]), k)] = True
    h = np.zeros((M, n))
    y = np.zeros((M, Wd.shape[1]))
    for m in range(M):
        idx = np.flatnonzero(keep[m])
        u = Wu[idx] @ x[m]                 # up rows of the kept neurons only
        h[m, idx] = a[m, idx] * u
        y[m] = h[m, idx] @ Wd[idx]         # down rows of the kept neurons only
    return dict(g=g, a=a, keep=keep, h=h, y=y)


def calibrate_gate(calib_x, Wg, p):
    """Threshold on |silu(g)| for target sparsity ``p``: the nearest-rank quantile
    (teal.calibrate_threshold) of the gate activations of the calibration tokens
    over every neuron, so that a fraction of at least p of the pool is dropped.

    Intra-expert summary, results: the threshold approach is tuned to a target
    sparsity (e.g. 85%) at which accuracy holds."""
    _, a = gate_activation(calib_x, Wg)
    return calibrate_threshold(a, p)
