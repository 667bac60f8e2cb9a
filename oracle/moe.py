"""Routed MoE layer with intra-expert activation sparsity, in fp64.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .teal import silu, dense_mlp, magnitude_mask
from .topk import value_topk


def router(x, Wr, top: int):
    """Router of one token: logits = x Wr; the ``top`` experts with the largest
    logits (ties to the smaller expert index); weights = softmax over the
    selected logits.

    Intra-expert summary, method section: routed experts are chosen by the
    router, shared experts are always active; the router logic is kept as is.
    Reading taken (the pages do not print the router): softmax renormalised over
    the selected experts.  Returns (ids in descending-logit order, weights).
    """
    x = np.asarray(x, dtype=np.float64)
    logits = x @ np.asarray(Wr, dtype=np.float64)
    sel = value_topk(logits, top)
    order = sel[np.lexsort((sel, -logits[sel]))]          # descending logit, ties by index
    z = logits[order]
    e = np.exp(z - z.max())
    return order, e / e.sum(), logits


def expert_sparse(x, Wgu_e, Wd_e, keep: int):
    """One routed expert on one token with intra-expert sparsity.

    Intra-expert summary, system implementation: the gate projection is run
    densely to score the neurons, the low-scoring neurons are skipped and only
    the active neurons' weights are gathered for the up/down work.  Reading
    taken (workload definition): gate and up are both dense, the score is
    |silu(g) * u|, and the ``keep`` largest (ties to the smaller index) reach
    the down projection.

    Wgu_e: ``[d_ff_e, 2, d_model]`` neuron-major; Wd_e: ``[d_ff_e, d_model]``.
    Returns (y_e, h, keep_idx).
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(Wgu_e, dtype=np.float64)
    g = W[:, 0, :] @ x
    u = W[:, 1, :] @ x
    h = silu(g) * u
    kidx = value_topk(np.abs(h), keep)
    y = h[kidx] @ np.asarray(Wd_e, dtype=np.float64)[kidx]
    return y, h, kidx


def expert_gate_score(x, Wgu_e, Wd_e, t):
    """One routed expert on one token with the gate-score keep rule.

    Intra-expert summary, system implementation: the gate projection runs densely
    and scores every neuron, one O(n) threshold pass masks the scores (no top-k
    sort), and only the active neurons' weights enter the up and down work.  TEAL
    slides, slides 5-6 (CATS): the score is |SiLU(x W_gate)|; W_up and W_down are
    pruned, the gate is not.

    Steps: ``g = W_gate x``, ``a = silu(g)``, keep j iff ``|a_j| > t`` (strict, t
    as fp32); for kept j ``u_j = W_up[j] . x`` and ``h_j = a_j u_j``; h is 0
    elsewhere; ``y_e = sum over kept j of h_j W_down[j]``.

    Wgu_e: ``[d_ff_e, 2, d_model]`` neuron-major; Wd_e: ``[d_ff_e, d_model]``.
    Returns (y_e, h, a, keep_idx).
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(Wgu_e, dtype=np.float64)
    a = silu(W[:, 0, :] @ x)
    kidx = np.flatnonzero(magnitude_mask(a, t))
    h = np.zeros(W.shape[0])
    h[kidx] = a[kidx] * (W[kidx, 1, :] @ x)        # up rows of the kept neurons only
    y = h[kidx] @ np.asarray(Wd_e, dtype=np.float64)[kidx]
    return y, h, a, kidx


def moe_layer_gate_score(x, w: dict, top: int, t):
    """The routed MoE layer of ``moe_layer`` with every routed expert under the
    gate-score keep rule (``expert_gate_score`` with threshold ``t``); the shared
    expert stays dense.  Returns (out, info) with per-token ids, weights, and per
    slot h, a and the kept neuron indices."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    T, d = x.shape
    out = np.zeros((T, d))
    info = []
    sgu = np.asarray(w["s_gate_up"], dtype=np.float64)
    for i in range(T):
        ids, wts, logits = router(x[i], w["w_router"], top)
        y = np.zeros(d)
        hs, as_, ks = [], [], []
        for e, we in zip(ids, wts):
            ye, h, a, kidx = expert_gate_score(x[i], w["w_gate_up"][e], w["w_down"][e], t)
            y += we * ye
            hs.append(h)
            as_.append(a)
            ks.append(kidx)
        y += dense_mlp(x[i], sgu[:, 0, :], sgu[:, 1, :], w["s_down"])
        out[i] = y
        info.append(dict(ids=ids, weights=wts, logits=logits, h=hs, a=as_, keep=ks))
    return out, info


def moe_layer(x, w: dict, top: int, keep: int):
    """``y_t = sum_j w_tj * expert_{e_tj}(x_t) + shared(x_t)`` for every token t.

    Intra-expert summary, method section: routed experts are sparsified inside,
    shared experts stay dense and are added unweighted.  ``w`` holds numpy fp64
    arrays: w_router [d, E], w_gate_up [E, d_ff_e, 2, d], w_down [E, d_ff_e, d],
    s_gate_up [d, 2, d_ff_s] (input-major), s_down [d_ff_s, d].
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    T = x.shape[0]
    d = x.shape[1]
    out = np.zeros((T, d))
    info = []
    for t in range(T):
        ids, wts, logits = router(x[t], w["w_router"], top)
        y = np.zeros(d)
        hs, ks = [], []
        for e, we in zip(ids, wts):
            ye, h, kidx = expert_sparse(x[t], w["w_gate_up"][e], w["w_down"][e], keep)
            y += we * ye
            hs.append(h)
            ks.append(kidx)
        sgu = np.asarray(w["s_gate_up"], dtype=np.float64)
        y += dense_mlp(x[t], sgu[:, 0, :], sgu[:, 1, :], w["s_down"])
        out[t] = y
        info.append(dict(ids=ids, weights=wts, logits=logits, h=hs, keep=ks))
    return out, info
