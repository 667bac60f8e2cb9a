"""Exact top-k and rank aggregation in plain numpy.

Test infrastructure only (see the package docstring).

Order conventions (readings, since the pages fix none of them):
* -0.0 equals +0.0; NaN sorts below every number, -inf included.
* top-k keeps the k largest by (value descending, index ascending), so among
  equal values the smaller index wins.
* ordinal rank: the largest value gets rank n, the smallest rank 1; among equal
  values the smaller index gets the higher rank (consistent with top-k).
"""
from __future__ import annotations

import numpy as np


def _clean(v: np.ndarray):
    v = np.asarray(v, dtype=np.float64).copy()
    nan = np.isnan(v)
    v[nan] = 0.0
    v[v == 0.0] = 0.0          # -0.0 -> +0.0
    return v, nan


def value_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices (ascending) of the k largest scores, ties to the smaller index.

    GLASS summary, section 2.2 (selection): the k neurons with the highest score
    form the pruning mask.  Intra-expert summary, method section: inside each
    routed expert the lowest-scoring neurons are zeroed, i.e. the highest k are
    kept.
    """
    v, nan = _clean(scores)
    n = v.size
    k = int(k)
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    idx = np.arange(n)
    # np.lexsort sorts by the last key first: NaN flag (0 before 1), then -v, then index.
    order = np.lexsort((idx, -v, nan.astype(np.int8)))
    return np.sort(order[:min(k, n)])


def ordinal_rank(v: np.ndarray) -> np.ndarray:
    """Ordinal ranks 1..n, largest value -> n; equal values: smaller index ranks higher.

    GLASS summary, section 2.2 (ranking): local and global importance scores are
    turned into ranks R^(l), R^(g) to remove their differences of scale and
    distribution.  Equivalently ``R_j = 1 + #{i : v_i < v_j or (v_i == v_j and i > j)}``.
    """
    w, nan = _clean(v)
    n = w.size
    idx = np.arange(n)
    # ascending by (not-NaN, value, -index): position p gets rank p + 1
    order = np.lexsort((-idx, w, (~nan).astype(np.int8)))
    r = np.empty(n, dtype=np.int64)
    r[order] = np.arange(1, n + 1)
    return r


def blend_weight_q16(lam: float) -> int:
    """lambda in 16-bit fixed point: round(lambda * 65536), half away from zero."""
    return int(np.floor(float(lam) * 65536.0 + 0.5))


def glass_scores(local: np.ndarray, prior: np.ndarray, lam: float) -> np.ndarray:
    """``S_j = (65536 - lq) R^(l)_j + lq R^(g)_j`` in int64, lq = round(lambda 65536).

    GLASS summary, section 2.2 (fusion rule): GLASS_j = (1 - lambda) R^(l)_j +
    lambda R^(g)_j, default lambda = 0.5.  Reading taken: lambda is carried in
    16-bit fixed point so the blend is integer and reproducible; S = 65536 *
    GLASS exactly whenever lambda is a multiple of 2^-16 (0.5 is).
    """
    lq = blend_weight_q16(lam)
    rl = ordinal_rank(local)
    rg = ordinal_rank(prior)
    return (65536 - lq) * rl + lq * rg


def glass_topk(local: np.ndarray, prior: np.ndarray, lam: float, k: int) -> np.ndarray:
    """Static neuron set: the k largest blended scores, ties to the smaller index.

    GLASS summary, section 2.2 (selection): the top-k neurons by GLASS score
    form the pruning mask that is then applied during decoding.
    """
    s = glass_scores(local, prior, lam).astype(np.float64)   # < 2^31: exact in fp64
    return value_topk(s, k)


def mask_from_index(idx: np.ndarray, n: int) -> np.ndarray:
    m = np.zeros(n, dtype=bool)
    m[np.asarray(idx, dtype=np.int64)] = True
    return m
