"""Static neuron-set FFN (GLASS) in fp64: local prompt signal and the masked decode MLP.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .teal import silu


def prompt_h(x_prompt, Wg, Wu):
    """FFN intermediate ``h = silu(x Wg) * (x Wu)`` of every prompt token (dense prefill).

    Wg, Wu given neuron-major ``[d_ff, d_model]`` (row j = neuron j's weights)."""
    x = np.asarray(x_prompt, dtype=np.float64)
    g = x @ np.asarray(Wg, dtype=np.float64).T
    u = x @ np.asarray(Wu, dtype=np.float64).T
    return silu(g) * u


def local_signal(h_prompt) -> np.ndarray:
    """Local importance of each FFN neuron: mean of |h| over the prompt tokens.

    GLASS summary, section 1 and 2.2: the local signal A^(l) is the activation
    of the prefill (prompt) stage.  Reading taken: the magnitude of the FFN
    intermediate (the down-projection input) averaged over the prompt tokens,
    with no per-token normalisation.
    """
    h = np.asarray(h_prompt, dtype=np.float64)
    return np.mean(np.abs(h), axis=0)


def neuron_set_mlp(x, Wg, Wu, Wd, idx):
    """SwiGLU restricted to the neurons in ``idx`` (all three matrices neuron-major
    ``[d_ff, d_model]``): ``y = sum_{j in idx} silu(x.Wg[j]) (x.Wu[j]) Wd[j]``.

    GLASS summary, section 2.2 and section 5 (efficiency): the static mask is
    applied for the whole decode, so only the kept neurons' weights are used.
    Glossary page: a neuron whose intermediate is zero skips its second-matrix
    row, and likewise its first-matrix column."""
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    Wg = np.asarray(Wg, dtype=np.float64)[idx]
    Wu = np.asarray(Wu, dtype=np.float64)[idx]
    Wd = np.asarray(Wd, dtype=np.float64)[idx]
    h = silu(x @ Wg.T) * (x @ Wu.T)
    return h @ Wd
