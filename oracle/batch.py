"""Batched decode with a static neuron set, and the batch-size switch, in fp64.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .teal import dense_mlp, swiglu_mlp_threshold

# Tokens from which the switch runs the dense path (measured on MI355X: from eight
# tokens on, the union of the tokens' threshold masks keeps nearly every row and
# the sparse launches cost more than the dense ones).
AUTO_DENSE_MIN_TOKENS = 8


def pack_neuron_set(Wgu, Wd, idx):
    """The kept neurons' weights as compact dense matrices: gate/up ``[d, 2, k]``
    (input-major, columns idx of every input row) and down ``[k, d]`` (rows idx).

    GLASS summary, section 2.2 and the edge-deployment discussion: a static mask
    keeps one compact subset of the weights resident for the whole decode.
    ``Wgu``: ``[d, 2, d_ff]`` input-major; ``Wd``: ``[d_ff, d]``."""
    idx = np.asarray(idx, dtype=np.int64)
    Wgu = np.asarray(Wgu, dtype=np.float64)
    return Wgu[:, :, idx], np.asarray(Wd, dtype=np.float64)[idx]


def static_set_mlp_batch(x, Wgu, Wd, idx):
    """``y_m = sum_{j in idx} silu(x_m . Wg[:, j]) (x_m . Wu[:, j]) Wd[j, :]`` for every
    token m of the batch (the same neuron set for every token)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    gu, dn = pack_neuron_set(Wgu, Wd, idx)
    return dense_mlp(x, gu[:, 0, :], gu[:, 1, :], dn)


def auto_mlp(x, Wgu, Wd, t_x, t_h):
    """The batch-size switch (Intra-expert summary, system implementation: sparse
    execution for low latency, dense execution for throughput, chosen by batch
    size): the threshold MLP for fewer than AUTO_DENSE_MIN_TOKENS tokens, the dense
    MLP from there on."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    Wgu = np.asarray(Wgu, dtype=np.float64)
    if x.shape[0] >= AUTO_DENSE_MIN_TOKENS:
        return dense_mlp(x, Wgu[:, 0, :], Wgu[:, 1, :], Wd)
    return swiglu_mlp_threshold(x, Wgu[:, 0, :], Wgu[:, 1, :], Wd, t_x, t_h)["y"]
