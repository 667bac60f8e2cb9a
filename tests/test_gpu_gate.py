"""GPU parity of the gate-score MLP (dense gate, |silu(g)| > t, up and down over the
kept neurons) against the fp64 oracle, stage by stage (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import gate, teal
from helpers import f64, rel_err, bits_to_bool, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_A = 1e-5     # silu(g): an fp32 dot product of d_model exact bf16/f16 products, then silu
TOL_Y = 2e-5     # a plain gather GEMV fed the GPU's own h


def _weights(d, f, dt="bf16", layer=0):
    W = datagen.mlp_weights_neuron_major(6, layer, d, f, dtype=dt)
    return W, asg.MLPWeights(W.to(DEV), None, L.AS_MLP_GATE_SCORE)


def _stagewise(X, W, w, t, check_e2e=True):
    """Run the GPU path with exports and check every stage against the oracle fed the
    GPU's own upstream tensors; returns (Y, debug dict, oracle dict)."""
    Y, dd = asg.as_sparse_swiglu_mlp(X.to(DEV), w, float("-inf"), float(t), debug=True)
    Wg, Wu, Wd = f64(W[:, 0]), f64(W[:, 1]), f64(W[:, 2])
    x = np.atleast_2d(f64(X))
    ref = gate.gate_score_mlp(x, Wg, Wu, Wd, t=np.float32(t))
    a = f64(dd["a"])
    # stage 1: the gate activation of every neuron
    assert rel_err(a, ref["a"]) < TOL_A
    # the keep mask is exact on the GPU's own scores (bits and counts)
    keep = teal.magnitude_mask(a, t)
    if "h_mask" in dd:
        assert np.array_equal(bits_to_bool(dd["h_mask"]["bits"], a.shape[1]), keep)
        assert dd["h_mask"]["nnz"].cpu().numpy().tolist() == keep.sum(axis=1).tolist()
    # h: a times the up dot product where kept, exactly 0 elsewhere
    h = f64(dd["h"])
    assert np.all(h[~keep] == 0.0)
    want_h = np.where(keep, a * (x @ Wu.T), 0.0)
    assert rel_err(h, want_h) < TOL_A
    # the down projection of the GPU's own h
    assert rel_err(Y, h @ Wd) < TOL_Y
    flips = int((keep != ref["keep"]).sum())
    e2e = rel_err(Y, ref["y"])
    print(f"keep {int(keep.sum())}/{keep.size}, flips vs fp64 chain {flips}, e2e {e2e:.2e}", flush=True)
    if check_e2e and flips == 0:
        assert e2e < 1e-4
    return Y, dd, ref


@pytest.mark.parametrize("M,d,f,dt,xdt", [(1, 256, 512, "bf16", "bf16"), (2, 256, 512, "f16", "f16"),
                                          (3, 512, 1024, "bf16", "f32"), (8, 384, 640, "bf16", "bf16"),
                                          (4, 1536, 320, "f16", "bf16"), (1, 4096, 1024, "bf16", "bf16")])
def test_gate_score_small(M, d, f, dt, xdt):
    """Several tiles of 16 neurons (ragged d_model chunks, d_ff not a multiple of 16*64),
    one to eight tokens, fp16/bf16 weights, bf16/f16/f32 inputs; t at the median score."""
    announce(f"gate score M={M} d={d} f={f} {dt}/{xdt}")
    W, w = _weights(d, f, dt)
    X = datagen.student_t((M, d), 60 + M + d, dtype=xdt)
    _, a = gate.gate_activation(f64(X), f64(W[:, 0]))
    t = float(np.float32(np.median(np.abs(a))))
    _stagewise(X, W, w, t)


def test_gate_score_limits():
    """t = -inf keeps every neuron (the dense SwiGLU); t = +inf keeps none (Y = 0
    exactly); FORCE_DENSE equals t = -inf bit for bit."""
    d, f = 256, 512
    W, w = _weights(d, f)
    X = datagen.student_t((2, d), 77).to(DEV)
    Wg, Wu, Wd = f64(W[:, 0]), f64(W[:, 1]), f64(W[:, 2])
    y_all = asg.as_sparse_swiglu_mlp(X, w, float("-inf"), float("-inf"))
    assert rel_err(y_all, teal.dense_mlp(f64(X), Wg.T, Wu.T, Wd)) < 1e-4
    y_dense = asg.as_sparse_swiglu_mlp(X, w, float("-inf"), 0.3, flags=L.AS_FLAG_FORCE_DENSE)
    assert torch.equal(y_dense, y_all)
    y_none = asg.as_sparse_swiglu_mlp(X, w, float("-inf"), float("inf"))
    assert torch.count_nonzero(y_none).item() == 0


def test_gate_score_rejects_input_threshold_and_large_batches():
    W, w = _weights(256, 512)
    X = datagen.student_t((1, 256), 5).to(DEV)
    with pytest.raises(L.ASError):
        asg.as_sparse_swiglu_mlp(X, w, 0.5, 0.1)
    X9 = datagen.student_t((9, 256), 5).to(DEV)
    with pytest.raises(L.ASError):
        asg.as_sparse_swiglu_mlp(X9, w, float("-inf"), 0.1)


@pytest.mark.parametrize("p", [0.5, 0.9])
def test_gate_score_llama_shape(p):
    """d_model 4096, d_ff 14336, bf16, batch 1 and 4: t calibrated on the GPU's own gate
    activations of 64 calibration tokens (nearest rank, as_calibrate_threshold),
    stage-wise parity on 4 decode tokens one at a time and on a batch of 4."""
    d, f = 4096, 14336
    announce(f"gate score llama p={p}")
    W, w = _weights(d, f)
    calib = datagen.student_t((64, d), datagen.seed_for(6, 0, "calib"))
    pool = []
    for b in range(0, 64, 8):
        _, dd = asg.as_sparse_swiglu_mlp(calib[b:b + 8].to(DEV), w, float("-inf"), float("-inf"), debug=True)
        pool.append(dd["a"].clone())
    t = float(asg.as_calibrate_threshold(torch.cat(pool), p).item())
    ref_t = gate.calibrate_gate(f64(calib), f64(W[:, 0]), p)
    print(f"t (GPU pool) {t:.6g}, t (fp64 pool) {float(ref_t):.6g}", flush=True)
    toks = datagen.student_t((4, d), datagen.seed_for(6, 0, "decode"))
    for i in range(4):
        _stagewise(toks[i:i + 1], W, w, t)
    _stagewise(toks, W, w, t)


def test_gate_score_deterministic():
    W, w = _weights(4096, 2048)
    X = datagen.student_t((2, 4096), 3).to(DEV)
    y1 = asg.as_sparse_swiglu_mlp(X, w, float("-inf"), 0.05)
    y2 = asg.as_sparse_swiglu_mlp(X, w, float("-inf"), 0.05)
    assert torch.equal(y1, y2)
