"""Pins for the gate-score (CATS / intra-expert) oracle (CPU only)."""
import itertools
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import gate


def _torch_dense(x, Wg, Wu, Wd):
    """Dense SwiGLU from torch's own silu, neuron-major weights."""
    x, Wg, Wu, Wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, Wg, Wu, Wd))
    return ((F.silu(x @ Wg.T) * (x @ Wu.T)) @ Wd).numpy()


def _weights(n=40, d=24, seed=7):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((3, d)), rng.standard_normal((n, d)) / 3,
            rng.standard_normal((n, d)) / 3, rng.standard_normal((n, d)) / 3)


def test_no_threshold_is_the_dense_swiglu():
    """t = -inf keeps every neuron: the result is the dense SwiGLU (torch's silu)."""
    x, Wg, Wu, Wd = _weights()
    r = gate.gate_score_mlp(x, Wg, Wu, Wd, t=-np.inf)
    assert r["keep"].all()
    np.testing.assert_allclose(r["y"], _torch_dense(x, Wg, Wu, Wd), rtol=1e-12, atol=1e-13)


def test_threshold_above_every_score_drops_everything():
    x, Wg, Wu, Wd = _weights()
    _, a = gate.gate_activation(x, Wg)
    t = np.float32(np.abs(a).max()) + np.float32(1.0)
    r = gate.gate_score_mlp(x, Wg, Wu, Wd, t=t)
    assert not r["keep"].any()
    assert np.all(r["y"] == 0.0) and np.all(r["h"] == 0.0)


def test_equals_dense_with_pruned_up_and_down_rows():
    """CATS prunes W_up and W_down, not the gate: zeroing the up and down rows of the
    dropped neurons in a dense torch SwiGLU gives the same output, token by token."""
    x, Wg, Wu, Wd = _weights(seed=11)
    _, a = gate.gate_activation(x, Wg)
    t = np.float32(np.median(np.abs(a)))
    r = gate.gate_score_mlp(x, Wg, Wu, Wd, t=t)
    assert 0 < r["keep"].sum() < r["keep"].size
    for m in range(x.shape[0]):
        kept = (np.abs(a[m]) > np.float64(t))[:, None]
        want = _torch_dense(x[m], Wg, np.where(kept, Wu, 0.0), np.where(kept, Wd, 0.0))
        np.testing.assert_allclose(r["y"][m], want, rtol=1e-12, atol=1e-13)


def test_keep_rule_is_the_magnitude_of_silu_of_the_gate():
    """g = (-3, 0.5, 2, -0.2): silu = (-0.1423, 0.3112, 1.7616, -0.0900).  At t = 0.12
    the kept set is {0, 1, 2}: |g| > t would also keep neuron 3, silu(g) > t would drop
    neuron 0, and |u| or |h| scores would pick by the up weights instead (neuron 3 has
    the largest up value)."""
    g = np.array([-3.0, 0.5, 2.0, -0.2])
    x = np.array([-3.0, 0.5, 2.0, 1.0])
    Wg = np.diag([1.0, 1.0, 1.0, -0.2])             # g = (x0, x1, x2, -0.2 x3)
    Wu = np.zeros((4, 4))
    Wu[:, 3] = [0.001, 5.0, 0.001, 9.0]             # u_j = Wu[j, 3] * x3
    Wd = np.eye(4)
    r = gate.gate_score_mlp(x, Wg, Wu, Wd, t=0.12)
    np.testing.assert_allclose(r["g"][0], g, rtol=0, atol=1e-15)
    silu = [v / (1.0 + math.exp(-v)) for v in g]
    np.testing.assert_allclose(r["a"][0], silu, rtol=1e-15)
    assert r["keep"][0].tolist() == [True, True, True, False]
    # h_j = a_j (x . Wu[j]) for the kept, 0 for neuron 3; y = h (Wd = identity)
    np.testing.assert_allclose(r["h"][0], [silu[0] * 0.001, silu[1] * 5.0, silu[2] * 0.001, 0.0], rtol=1e-15)
    np.testing.assert_allclose(r["y"][0], r["h"][0], rtol=0)


def test_permuting_neurons_permutes_keep_and_h_and_keeps_y():
    x, Wg, Wu, Wd = _weights(n=33, d=20, seed=5)
    perm = np.random.default_rng(1).permutation(33)
    _, a = gate.gate_activation(x, Wg)
    t = np.float32(np.quantile(np.abs(a), 0.6))
    r = gate.gate_score_mlp(x, Wg, Wu, Wd, t=t)
    q = gate.gate_score_mlp(x, Wg[perm], Wu[perm], Wd[perm], t=t)
    assert np.array_equal(q["keep"], r["keep"][:, perm])
    np.testing.assert_allclose(q["h"], r["h"][:, perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(q["y"], r["y"], rtol=1e-12, atol=1e-13)


def test_topk_keeps_the_k_largest_scores_brute_force():
    """k = 3 of 7 neurons: the kept set has the largest sum of |a| over all C(7, 3)
    subsets (scores distinct), and the output is the dense SwiGLU on that set."""
    rng = np.random.default_rng(21)
    d, n = 6, 7
    x = rng.standard_normal(d)
    Wg, Wu, Wd = (rng.standard_normal((n, d)) for _ in range(3))
    r = gate.gate_score_mlp(x, Wg, Wu, Wd, k=3)
    a = np.abs(r["a"][0])
    best = max(itertools.combinations(range(n), 3), key=lambda S: sum(a[list(S)]))
    assert sorted(np.flatnonzero(r["keep"][0]).tolist()) == sorted(best)
    idx = list(best)
    np.testing.assert_allclose(r["y"][0], _torch_dense(x, Wg[idx], Wu[idx], Wd[idx]), rtol=1e-12, atol=1e-13)


def test_tokens_are_independent():
    x, Wg, Wu, Wd = _weights(seed=3)
    r = gate.gate_score_mlp(x, Wg, Wu, Wd, t=0.1)
    for m in range(x.shape[0]):
        s = gate.gate_score_mlp(x[m], Wg, Wu, Wd, t=0.1)
        assert np.array_equal(s["keep"][0], r["keep"][m])
        np.testing.assert_allclose(s["y"][0], r["y"][m], rtol=1e-12, atol=1e-13)


def test_calibration_reaches_the_target_sparsity_by_nearest_rank():
    """On the calibration pool itself, at least ceil(p n) of the n gate activations
    satisfy |a| <= t, and t is the smallest fp32 that does so (the next fp32 below
    it leaves fewer than ceil(p n)): the nearest-rank p-quantile rounded up to fp32."""
    rng = np.random.default_rng(9)
    calib = rng.standard_normal((17, 24))
    Wg = rng.standard_normal((50, 24)) / 4
    _, a = gate.gate_activation(calib, Wg)
    v = np.abs(a).ravel()
    for p in (0.1, 0.5, 0.85, 0.9):
        t32 = gate.calibrate_gate(calib, Wg, p)
        below = np.float64(np.nextafter(t32, np.float32(-np.inf)))
        r = math.ceil(p * v.size)
        assert (v <= np.float64(t32)).sum() >= r
        assert (v <= below).sum() < r
