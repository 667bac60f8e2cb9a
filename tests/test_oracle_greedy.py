"""Pins for the block-wise greedy sparsity allocation oracle (CPU only)."""
import itertools

import numpy as np

from oracle import greedy


def _convex_curves(nb, nl, seed):
    """Increasing, convex error curves (increments positive and growing)."""
    rng = np.random.default_rng(seed)
    inc = np.sort(rng.uniform(0.01, 1.0, (nb, nl - 1)), axis=1) * rng.uniform(0.2, 3.0, (nb, 1))
    return np.concatenate([np.zeros((nb, 1)), np.cumsum(inc, axis=1)], axis=1)


def test_greedy_is_optimal_on_convex_curves_brute_force():
    """Separable convex costs: raising the cheapest block one step at a time reaches
    the least total error among all allocations with the same number of steps
    (brute force over every level vector)."""
    for seed in range(6):
        nb, nl, step = 4, 5, 0.1
        err = _convex_curves(nb, nl, seed)
        for target in (0.05, 0.1, 0.2, 0.25):
            lev = greedy.greedy_allocate(err, np.ones(nb), step, target)
            k = int(lev.sum())
            assert abs(k * step / nb - target) < 1e-9 or k * step / nb >= target
            best = min(sum(err[b, c[b]] for b in range(nb))
                       for c in itertools.product(range(nl), repeat=nb) if sum(c) == k)
            got = sum(err[b, lev[b]] for b in range(nb))
            assert abs(got - best) < 1e-12


def test_identical_blocks_get_a_uniform_allocation_smaller_index_first():
    err = np.tile(np.array([0.0, 1.0, 3.0, 6.0, 10.0]), (5, 1))
    lev = greedy.greedy_allocate(err, np.ones(5), 0.1, 0.16)     # 8 steps over 5 blocks
    assert lev.tolist() == [2, 2, 2, 1, 1]


def test_a_free_block_is_raised_to_its_last_level_first():
    err = np.array([[0.0, 1.0, 2.0, 3.0], [0.0, 0.0, 0.0, 0.0], [0.0, 0.5, 1.5, 3.0]])
    lev = greedy.greedy_allocate(err, np.ones(3), 0.25, 0.5)     # 6 steps
    assert lev[1] == 3
    # then b2 (+0.5), then ties of +1.0 go to the smaller index, b0, twice
    assert lev.sum() == 6 and lev.tolist() == [2, 3, 1]


def test_limits_and_weighted_target_is_met_minimally():
    """Target 0 keeps every block dense, target 1 takes every block to its last
    level; a weighted target is met and overshot by less than one step of the
    heaviest block (the allocation stops at the first step that meets it)."""
    err = _convex_curves(3, 6, 11)
    assert greedy.greedy_allocate(err, np.ones(3), 0.2, 0.0).tolist() == [0, 0, 0]
    assert greedy.greedy_allocate(err, np.ones(3), 0.2, 1.0).tolist() == [5, 5, 5]
    w = np.array([1.0, 3.0, 0.5])
    for target in (0.1, 0.33, 0.5, 0.77):
        lev = greedy.greedy_allocate(err, w, 0.2, target)
        overall = (w * lev * 0.2).sum() / w.sum()
        assert overall >= target - 1e-12
        assert overall - w.max() * 0.2 / w.sum() < target
