"""GPU parity of batched static-set decode (compact packed weights) and the
batch-size switch (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import batch
from helpers import f64, rel_err, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _weights(d, f, layer=0):
    wgu, wd = datagen.mlp_weights_input_major(10, layer, datagen.MLPShape(d, f, "bf16"))
    return wgu, wd, asg.MLPWeights(wgu.to(DEV), wd.to(DEV))


def _idx(f, k, seed):
    return np.sort(np.random.default_rng(seed).choice(f, k, replace=False)).astype(np.int32)


def test_pack_is_an_exact_copy():
    d, f, k = 4096, 14336, 7168
    wgu, wd, w = _weights(d, f)
    I = _idx(f, k, 1)
    p = asg.as_pack_neuron_set(w, torch.from_numpy(I).to(DEV))
    gu, dn = batch.pack_neuron_set(f64(wgu), f64(wd), I)
    assert np.array_equal(f64(p.w_gate_up), gu) and np.array_equal(f64(p.w_down), dn)


@pytest.mark.parametrize("M", [8, 16, 32, 64])
def test_batched_static_set_mlp(M):
    """The packed set's dense SwiGLU over a batch (groups of 16 tokens past 16)
    against the fp64 static-set MLP."""
    announce(f"static set batch M={M}")
    d, f, k = 4096, 14336, 7168
    wgu, wd, w = _weights(d, f, layer=1)
    I = _idx(f, k, M)
    p = asg.as_pack_neuron_set(w, torch.from_numpy(I).to(DEV))
    X = datagen.student_t((M, d), 40 + M)
    Y = asg.as_sparse_swiglu_mlp(X.to(DEV), p, flags=L.AS_FLAG_FORCE_DENSE)
    ref = batch.static_set_mlp_batch(f64(X), f64(wgu), f64(wd), I)
    assert rel_err(Y, ref) < 1e-4
    assert torch.equal(Y, asg.as_sparse_swiglu_mlp(X.to(DEV), p, flags=L.AS_FLAG_FORCE_DENSE))


def test_more_than_16_tokens_run_as_groups_of_16():
    """M = 37 threshold-mode tokens give the bits of the three group calls."""
    d, f = 1024, 4096
    wgu, wd, w = _weights(d, f, layer=2)
    X = datagen.student_t((37, d), 9).to(DEV)
    t_x, t_h = 0.8, 0.01
    Y = asg.as_sparse_swiglu_mlp(X, w, t_x, t_h)
    parts = [asg.as_sparse_swiglu_mlp(X[a:b], w, t_x, t_h) for a, b in ((0, 16), (16, 32), (32, 37))]
    assert torch.equal(Y, torch.cat(parts))


@pytest.mark.parametrize("M", [1, 4, 7, 8, 12])
def test_auto_switch(M):
    d, f = 1024, 4096
    wgu, wd, w = _weights(d, f, layer=3)
    X = datagen.student_t((M, d), 11 + M).to(DEV)
    y_auto = asg.as_sparse_swiglu_mlp(X, w, 0.8, 0.01, flags=L.AS_FLAG_AUTO)
    want = (asg.as_sparse_swiglu_mlp(X, w, 0.8, 0.01, flags=L.AS_FLAG_FORCE_DENSE)
            if M >= L.AS_AUTO_DENSE_MIN_TOKENS else asg.as_sparse_swiglu_mlp(X, w, 0.8, 0.01))
    assert torch.equal(y_auto, want)
    ref = batch.auto_mlp(f64(X), f64(wgu), f64(wd), 0.8, 0.01)
    assert rel_err(y_auto, ref) < 2e-3
