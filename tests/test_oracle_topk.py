"""Pins for the top-k and rank-blend oracle (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import topk


def _parse(v):
    return np.array([float(s) for s in v], dtype=np.float64)


def _beats(a_val, a_idx, b_val, b_idx):
    """a precedes b in the (value desc, index asc) order; NaN below all, -0 == +0."""
    an, bn = np.isnan(a_val), np.isnan(b_val)
    if an != bn:
        return bn
    if not an and a_val != b_val:
        return a_val > b_val
    return a_idx < b_idx


def _brute_topk(v, k):
    n = len(v)
    sols = []
    for S in itertools.combinations(range(n), k):
        Sset = set(S)
        if all(_beats(v[i], i, v[j], j) for i in S for j in range(n) if j not in Sset):
            sols.append(list(S))
    assert len(sols) == 1
    return sols[0]


def test_hand_cases(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "topk_cases.json")))
    for c in g["value_topk"]:
        assert topk.value_topk(_parse(c["scores"]), c["k"]).tolist() == c["idx"], c
    for c in g["rank"]:
        assert topk.ordinal_rank(np.array(c["v"])).tolist() == c["R"], c
    for c in g["blend"]:
        rl = topk.ordinal_rank(np.array(c["local"]))
        rg = topk.ordinal_rank(np.array(c["prior"]))
        assert (rl + rg).tolist() == c["sum_ranks"]
        S = topk.glass_scores(np.array(c["local"]), np.array(c["prior"]), c["lambda"])
        assert S.tolist() == [32768 * s for s in c["sum_ranks"]]
        for k, idx in c["k"].items():
            assert topk.glass_topk(np.array(c["local"]), np.array(c["prior"]), c["lambda"], int(k)).tolist() == idx


@pytest.mark.parametrize("seed", range(25))
def test_value_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    v = rng.integers(-3, 4, size=n).astype(np.float64)      # many ties
    if seed % 3 == 0:
        v[rng.integers(0, n)] = np.nan
    if seed % 4 == 0:
        v[rng.integers(0, n)] = -0.0
    for k in range(0, n + 1):
        assert topk.value_topk(v, k).tolist() == sorted(_brute_topk(v, k))


def test_all_equal_gives_first_k():
    assert topk.value_topk(np.full(100, 0.25), 37).tolist() == list(range(37))


@pytest.mark.parametrize("seed", range(10))
def test_rank_is_permutation_and_order_preserving(seed):
    rng = np.random.default_rng(seed)
    n = 500
    v = np.round(rng.random(n), 2)                            # forced collisions
    R = topk.ordinal_rank(v)
    assert sorted(R.tolist()) == list(range(1, n + 1))
    for _ in range(2000):
        i, j = rng.integers(0, n, 2)
        if v[i] < v[j]:
            assert R[i] < R[j]
        elif v[i] == v[j] and i < j:
            assert R[i] > R[j]


def test_rank_counts_definition_small():
    # brute count of elements ranked below, on a tiny vector with ties
    v = np.array([0.3, 0.1, 0.3, 0.2, 0.1])
    R = topk.ordinal_rank(v)
    assert R.tolist() == [5, 2, 4, 3, 1]


@pytest.mark.parametrize("seed", range(8))
def test_lambda_endpoints_reduce_to_single_signal(seed):
    rng = np.random.default_rng(100 + seed)
    n = 300
    local = np.round(rng.random(n), 3)
    prior = rng.random(n).astype(np.float32).astype(np.float64)
    for k in (1, 50, 150, 299, 300):
        # lambda = 0 is the prompt-only mask, lambda = 1 the global-prior-only mask
        assert topk.glass_topk(local, prior, 0.0, k).tolist() == topk.value_topk(local, k).tolist()
        assert topk.glass_topk(local, prior, 1.0, k).tolist() == topk.value_topk(prior, k).tolist()


def test_blend_half_is_rank_sum_order():
    rng = np.random.default_rng(7)
    n = 64
    local, prior = rng.random(n), rng.random(n)
    S = topk.glass_scores(local, prior, 0.5)
    rs = topk.ordinal_rank(local) + topk.ordinal_rank(prior)
    assert np.array_equal(S, 32768 * rs)
    assert topk.blend_weight_q16(0.5) == 32768 and topk.blend_weight_q16(1.0) == 65536
