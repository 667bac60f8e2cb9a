"""Pins for the attribution-selection oracle (CPU only)."""
import itertools
import math

import numpy as np

from oracle import attrib


def test_corrected_gxo_by_hand():
    """x = (1, -2, 0.5), grad = (3, 4, 0): |grad| = 5, score = g x + |x| * 5 / 2."""
    s = attrib.corrected_gxo([1.0, -2.0, 0.5], [3.0, 4.0, 0.0])
    assert s.tolist() == [[3.0 + 2.5, -8.0 + 5.0, 0.0 + 1.25]]


def test_corrected_gxo_special_cases():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 30))
    assert np.all(attrib.corrected_gxo(x, np.zeros_like(x)) == 0)
    # one-hot gradient: the correction is |x_i| / 2 for every neuron, plus g x at the hot one
    g = np.zeros_like(x)
    g[:, 7] = 2.0
    s = attrib.corrected_gxo(x, g)
    want = np.abs(x) * 1.0
    want[:, 7] += 2.0 * x[:, 7]
    np.testing.assert_allclose(s, want, rtol=1e-15)
    # rows are independent layers
    np.testing.assert_allclose(attrib.corrected_gxo(x[2], g[2])[0], s[2], rtol=0)


def test_top_fraction_brute_force_and_count():
    rng = np.random.default_rng(5)
    s = np.round(rng.standard_normal((3, 9)), 1)            # ties
    keep = attrib.top_fraction(s, 1, 3)                      # k = ceil(9 / 3) = 3
    for r in range(3):
        best = max(itertools.combinations(range(9), 3),
                   key=lambda S: (sorted(s[r, list(S)], reverse=True), [-i for i in S]))
        assert sorted(np.flatnonzero(keep[r]).tolist()) == sorted(best)
    assert attrib.fraction_count(10, 3, 10) == 3
    assert attrib.fraction_count(10, 31, 100) == 4          # 3.1 rounds up
    assert attrib.fraction_count(7, 0, 1) == 0 and attrib.fraction_count(7, 1, 1) == 7
    assert attrib.fraction_count(14336, 2, 5) == math.ceil(0.4 * 14336)


def test_head_masked_gemv_equals_dense_with_zeroed_blocks():
    rng = np.random.default_rng(9)
    nh, hd, N = 6, 8, 20
    x = rng.standard_normal(nh * hd)
    W = rng.standard_normal((nh * hd, N))
    heads = [0, 3, 4]
    mask = np.zeros(nh * hd)
    for h in heads:
        mask[h * hd:(h + 1) * hd] = 1
    np.testing.assert_allclose(attrib.head_masked_gemv(x, W, heads, hd), (x * mask) @ W, rtol=1e-12, atol=1e-13)
    assert np.all(attrib.head_masked_gemv(x, W, [], hd) == 0)
    np.testing.assert_allclose(attrib.head_masked_gemv(x, W, range(nh), hd), x @ W, rtol=1e-12, atol=1e-13)
