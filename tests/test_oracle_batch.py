"""Pins for the static-set batch and switch oracle (CPU only)."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import batch, glass, teal


def _w(d=24, f=40, seed=1):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((d, 2, f)) / 4, rng.standard_normal((f, d)) / 4


def test_packed_set_equals_the_neuron_set_mlp_on_neuron_major_weights():
    """The compact input-major matrices give the neuron-set MLP of the GLASS oracle
    (neuron-major weights, another layout and code path), token by token."""
    Wgu, Wd = _w()
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 24))
    idx = np.array([0, 3, 4, 17, 39])
    y = batch.static_set_mlp_batch(x, Wgu, Wd, idx)
    ref = glass.neuron_set_mlp(x, Wgu[:, 0, :].T, Wgu[:, 1, :].T, Wd, idx)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_all_neurons_is_the_dense_mlp_and_none_is_zero():
    Wgu, Wd = _w(seed=3)
    x = np.random.default_rng(4).standard_normal((3, 24))
    xt = torch.from_numpy(x)
    ref = ((F.silu(xt @ torch.from_numpy(Wgu[:, 0, :])) * (xt @ torch.from_numpy(Wgu[:, 1, :])))
           @ torch.from_numpy(Wd)).numpy()
    np.testing.assert_allclose(batch.static_set_mlp_batch(x, Wgu, Wd, np.arange(40)), ref, rtol=1e-12, atol=1e-13)
    assert np.all(batch.static_set_mlp_batch(x, Wgu, Wd, np.array([], dtype=np.int64)) == 0)


def test_pack_layout():
    Wgu, Wd = _w(seed=5)
    idx = np.array([2, 7, 9])
    gu, dn = batch.pack_neuron_set(Wgu, Wd, idx)
    assert gu.shape == (24, 2, 3) and dn.shape == (3, 24)
    assert np.array_equal(gu[5, 1, 2], Wgu[5, 1, 9]) and np.array_equal(dn[1], Wd[7])


def test_switch_follows_the_batch_size():
    Wgu, Wd = _w(seed=6)
    rng = np.random.default_rng(7)
    for M in (1, 7, 8, 12):
        x = rng.standard_normal((M, 24))
        y = batch.auto_mlp(x, Wgu, Wd, 0.5, 0.01)
        dense = teal.dense_mlp(x, Wgu[:, 0, :], Wgu[:, 1, :], Wd)
        sparse = teal.swiglu_mlp_threshold(x, Wgu[:, 0, :], Wgu[:, 1, :], Wd, 0.5, 0.01)["y"]
        want = dense if M >= batch.AUTO_DENSE_MIN_TOKENS else sparse
        assert np.array_equal(y, want)
        assert not np.allclose(dense, sparse)
