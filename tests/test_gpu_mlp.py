"""GPU parity of the sparse SwiGLU MLP (threshold and static neuron-set modes),
checked stage by stage against the fp64 oracle (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import teal, glass
from helpers import TOL, f64, rel_err, bits_to_bool, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

_CACHE = {}


def _mlp(cfg, shape):
    key = (cfg, shape)
    if key not in _CACHE:
        wgu, wd = datagen.mlp_weights_input_major(cfg, 0, shape)
        _CACHE.clear()
        _CACHE[key] = dict(wgu=wgu, wd=wd, Wg=f64(wgu[:, 0, :]), Wu=f64(wgu[:, 1, :]), Wd=f64(wd),
                           dev=asg.MLPWeights(wgu.to(DEV), wd.to(DEV)))
    return _CACHE[key]


def _check_stagewise(x, w, t_x, t_h, M):
    """Stage-wise parity: x mask exact; h within tolerance; h mask exact on the GPU's h;
    y within tolerance of the oracle's down stage fed the GPU's h."""
    y, dbg = asg.as_sparse_swiglu_mlp(x.to(DEV), w["dev"], t_x, t_h, debug=True)
    X = f64(x)
    d = X.shape[1]
    f = w["Wg"].shape[1]
    m1 = teal.magnitude_mask(X, t_x)
    assert np.array_equal(bits_to_bool(dbg["x_mask"]["bits"], d), m1)
    assert dbg["x_mask"]["nnz"].cpu().numpy().tolist() == m1.sum(axis=1).tolist()
    r = teal.swiglu_mlp_threshold(X, w["Wg"], w["Wu"], w["Wd"], t_x, t_h)
    h_gpu = f64(dbg["h"])
    # h: exact products, fp32 sums, fp32 SwiGLU; y: a plain GEMV of the GPU's h, whose
    # matrix-core path (more than 8 tokens) carries each fp32 activation as bf16 hi +
    # lo (2^-17 relative per term)
    tol_y = 2e-5 if M <= 8 else 2e-4
    eh = rel_err(h_gpu, r["h"])
    assert eh < 1e-5, eh
    m2 = teal.magnitude_mask(h_gpu, t_h)
    assert np.array_equal(bits_to_bool(dbg["h_mask"]["bits"], f), m2)
    assert dbg["h_mask"]["nnz"].cpu().numpy().tolist() == m2.sum(axis=1).tolist()
    y_ref = teal.down_stage(h_gpu, w["Wd"], t_h)
    err = rel_err(y, y_ref)
    assert err < tol_y, err
    flips = int((m2 != r["m2"]).sum())
    e2e = rel_err(y, r["y"])
    if flips == 0:
        assert e2e < TOL
    # without exports, several tokens take the range-masked gate/up stage
    y_plain = asg.as_sparse_swiglu_mlp(x.to(DEV), w["dev"], t_x, t_h)
    assert rel_err(y_plain, f64(y)) < TOL
    return dict(err=err, e2e=e2e, flips=flips, sparsity_x=1 - m1.mean(), sparsity_h=1 - m2.mean())


def test_mlp_small_fp16_workload():
    """SwiGLU 512 -> 2048 -> 512, fp16 weights, Laplace inputs, 50% thresholds from 256
    calibration vectors, 64 decode tokens one at a time and batched by 8."""
    shape = datagen.CFG1
    w = _mlp(1, shape)
    calib = datagen.laplace((256, shape.d_model), datagen.seed_for(1, 0, "calib"), dtype="f16")
    t_x, t_h, _ = teal.calibrate_mlp(f64(calib), w["Wg"], w["Wu"], 0.5, 0.5)
    toks = datagen.laplace((64, shape.d_model), datagen.seed_for(1, 0, "decode"), dtype="f16")
    for i in range(64):
        announce(f"mlp small token {i}")
        _check_stagewise(toks[i:i + 1], w, float(t_x), float(t_h), 1)
    for b in range(0, 64, 8):
        announce(f"mlp small batch {b}")
        _check_stagewise(toks[b:b + 8], w, float(t_x), float(t_h), 8)


@pytest.mark.parametrize("s", datagen.CFG2_SWEEP)
def test_mlp_llama_sweep(s):
    """Llama-3-8B-shaped MLP (4096 -> 14336 -> 4096, bf16), Student-t(3) inputs, thresholds
    calibrated at sparsity s on both inputs, in the launch configuration the benchmark times."""
    shape = datagen.CFG2
    w = _mlp(2, shape)
    calib = datagen.student_t((256, shape.d_model), datagen.seed_for(2, 0, "calib"))
    t_x, t_h, _ = teal.calibrate_mlp(f64(calib), w["Wg"], w["Wu"], s, s)
    toks = datagen.student_t((4, shape.d_model), datagen.seed_for(2, 0, "decode"))
    for i in range(4):
        announce(f"mlp llama s={s} token {i}")
        r = _check_stagewise(toks[i:i + 1], w, float(t_x), float(t_h), 1)
        print(r, flush=True)


@pytest.mark.parametrize("M", [9, 16])
def test_mlp_batched_mfma(M):
    """Threshold MLP for 9..16 tokens on the matrix cores (Llama-3-8B shape, 50%)."""
    announce(f"mlp mfma M={M}")
    shape = datagen.CFG2
    w = _mlp(2, shape)
    calib = datagen.student_t((256, shape.d_model), datagen.seed_for(2, 0, "calib"))
    t_x, t_h, _ = teal.calibrate_mlp(f64(calib), w["Wg"], w["Wu"], 0.5, 0.5)
    toks = datagen.student_t((M, shape.d_model), datagen.seed_for(2, 1, "decode"))
    r = _check_stagewise(toks, w, float(t_x), float(t_h), M)
    print(r, flush=True)
    y = asg.as_sparse_swiglu_mlp(toks.to(DEV), w["dev"], 5.0, 5.0, flags=L.AS_FLAG_FORCE_DENSE)
    assert rel_err(y, teal.dense_mlp(f64(toks), w["Wg"], w["Wu"], w["Wd"])) < TOL


def test_mlp_dense_baseline_matches_dense_oracle():
    announce("mlp dense baseline")
    shape = datagen.CFG2
    w = _mlp(2, shape)
    x = datagen.student_t((1, shape.d_model), 77)
    y = asg.as_sparse_swiglu_mlp(x.to(DEV), w["dev"], 5.0, 5.0, flags=L.AS_FLAG_FORCE_DENSE)
    ref = teal.dense_mlp(f64(x), w["Wg"], w["Wu"], w["Wd"])
    assert rel_err(y, ref) < TOL
    # sparsity 0 (t = -inf on both inputs) computes the same function
    y0 = asg.as_sparse_swiglu_mlp(x.to(DEV), w["dev"], float("-inf"), float("-inf"))
    assert rel_err(y0, ref) < TOL


@pytest.mark.parametrize("cfg,M", [(1, 1), (2, 1), (1, 4), (2, 8), (2, 16)])
def test_mlp_h_mask_count_and_reproducibility(cfg, M):
    """The h-mask count export equals the popcount of the exported bits (and the
    oracle's count on the GPU's h), and the whole call is bitwise reproducible: the
    same y, h and masks on a second call with the same workspace (the one-token path
    sums the unsummed gate/up partials in the down prologue; several tokens combine
    in the gate/up launch; 16 tokens run on the matrix cores)."""
    announce(f"mlp h nnz + run twice cfg={cfg} M={M}")
    shape = datagen.CFG1 if cfg == 1 else datagen.CFG2
    w = _mlp(cfg, shape)
    gen = datagen.laplace if cfg == 1 else datagen.student_t
    kw = dict(dtype="f16") if cfg == 1 else {}
    calib = gen((64, shape.d_model), datagen.seed_for(cfg, 0, "calib"), **kw)
    x = gen((M, shape.d_model), datagen.seed_for(cfg, 5, "decode"), **kw).to(DEV)
    t_x, t_h, _ = teal.calibrate_mlp(f64(calib), w["Wg"], w["Wu"], 0.5, 0.5)
    y1, d1 = asg.as_sparse_swiglu_mlp(x, w["dev"], float(t_x), float(t_h), debug=True)
    y2, d2 = asg.as_sparse_swiglu_mlp(x, w["dev"], float(t_x), float(t_h), debug=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(d1["h"], d2["h"])
    for k in ("bits", "nnz"):
        assert torch.equal(d1["h_mask"][k], d2["h_mask"][k])
        assert torch.equal(d1["x_mask"][k], d2["x_mask"][k])
    f = shape.d_ff
    m2 = teal.magnitude_mask(f64(d1["h"]), t_h)
    assert np.array_equal(bits_to_bool(d1["h_mask"]["bits"], f), m2)
    assert d1["h_mask"]["nnz"].cpu().numpy().tolist() == m2.sum(axis=1).tolist()


@pytest.mark.parametrize("cfg,M", [(2, 1), (2, 4), (2, 16), (1, 1), (1, 3)])
def test_mlp_atomic_splitk(cfg, M):
    """AS_FLAG_ATOMIC_SPLITK in the threshold MLP: the down stage adds into fp32 Y with
    atomics (the gate/up launch clears Y first, so a NaN-filled Y is overwritten).  y is
    checked against the oracle's down stage fed the GPU's h, and against the
    deterministic path; with AS_FLAG_ACCUMULATE it lands on Y's contents."""
    announce(f"mlp atomic split-K cfg={cfg} M={M}")
    shape = datagen.CFG1 if cfg == 1 else datagen.CFG2
    w = _mlp(cfg, shape)
    if cfg == 1:
        calib = datagen.laplace((64, shape.d_model), datagen.seed_for(1, 0, "calib"), dtype="f16")
        toks = datagen.laplace((M, shape.d_model), datagen.seed_for(1, 4, "decode"), dtype="f16")
    else:
        calib = datagen.student_t((64, shape.d_model), datagen.seed_for(2, 0, "calib"))
        toks = datagen.student_t((M, shape.d_model), datagen.seed_for(2, 4, "decode"))
    t_x, t_h, _ = teal.calibrate_mlp(f64(calib), w["Wg"], w["Wu"], 0.5, 0.5)
    t_x, t_h = float(t_x), float(t_h)
    xd = toks.to(DEV)
    Y = torch.full((M, shape.d_model), float("nan"), device=DEV)
    _, dbg = asg.as_sparse_swiglu_mlp(xd, w["dev"], t_x, t_h, flags=L.AS_FLAG_ATOMIC_SPLITK, Y=Y, debug=True)
    y_ref = teal.down_stage(f64(dbg["h"]), w["Wd"], t_h)
    assert rel_err(Y, y_ref) < TOL
    Y2 = torch.full((M, shape.d_model), float("nan"), device=DEV)
    asg.as_sparse_swiglu_mlp(xd, w["dev"], t_x, t_h, flags=L.AS_FLAG_ATOMIC_SPLITK, Y=Y2)
    y_det = asg.as_sparse_swiglu_mlp(xd, w["dev"], t_x, t_h)
    assert rel_err(Y2, f64(y_det)) < 1e-5
    Y0 = torch.randn(M, shape.d_model, device=DEV)
    Y1 = Y0.clone()
    asg.as_sparse_swiglu_mlp(xd, w["dev"], t_x, t_h, flags=L.AS_FLAG_ATOMIC_SPLITK | L.AS_FLAG_ACCUMULATE, Y=Y1)
    assert rel_err(Y1, f64(Y0) + f64(y_det)) < 1e-5
    yd = asg.as_sparse_swiglu_mlp(xd, w["dev"], flags=L.AS_FLAG_FORCE_DENSE | L.AS_FLAG_ATOMIC_SPLITK)
    assert rel_err(yd, teal.dense_mlp(f64(toks), w["Wg"], w["Wu"], w["Wd"])) < TOL


def test_neuron_set_atomic_splitk():
    announce("neuron-set atomic split-K")
    d, f, n_act = 512, 2048, 777
    W, Wg, Wu, Wd = _neuron_major(d, f, 9)
    idx = np.sort(np.random.default_rng(5).choice(f, size=n_act, replace=False)).astype(np.int32)
    x = datagen.student_t((2, d), 57)
    w = asg.MLPWeights(W.to(DEV), None, L.AS_MLP_NEURON_SET)
    Y = torch.full((2, d), float("nan"), device=DEV)
    asg.as_sparse_swiglu_mlp(x.to(DEV), w, neuron_idx=torch.from_numpy(idx).to(DEV),
                             flags=L.AS_FLAG_ATOMIC_SPLITK, Y=Y)
    assert rel_err(Y, glass.neuron_set_mlp(f64(x), Wg, Wu, Wd, idx)) < TOL


def test_mlp_determinism_and_edges():
    announce("mlp determinism")
    shape = datagen.CFG1
    w = _mlp(1, shape)
    x = datagen.laplace((1, shape.d_model), 91, dtype="f16").to(DEV)
    y1 = asg.as_sparse_swiglu_mlp(x, w["dev"], 0.7, 0.01)
    y2 = asg.as_sparse_swiglu_mlp(x, w["dev"], 0.7, 0.01)
    assert torch.equal(y1, y2)
    # everything masked at the input: y == 0
    y = asg.as_sparse_swiglu_mlp(x, w["dev"], 1e30, 0.0)
    assert torch.count_nonzero(y).item() == 0
    # everything masked at h: y == 0
    y = asg.as_sparse_swiglu_mlp(x, w["dev"], 0.5, 1e30)
    assert torch.count_nonzero(y).item() == 0


def _neuron_major(d, f, seed):
    W = datagen.mlp_weights_neuron_major(4, seed, d, f)
    return W, f64(W[:, 0]), f64(W[:, 1]), f64(W[:, 2])


@pytest.mark.parametrize("d,f,n_act,M", [(512, 2048, 1024, 1), (512, 2048, 777, 3), (4096, 14336, 7168, 1),
                                         (4096, 14336, 1, 1), (4096, 14336, 0, 1)])
def test_neuron_set_mlp(d, f, n_act, M):
    announce(f"neuron-set d={d} f={f} n={n_act} M={M}")
    W, Wg, Wu, Wd = _neuron_major(d, f, d + n_act)
    rng = np.random.default_rng(n_act + 1)
    idx = np.sort(rng.choice(f, size=n_act, replace=False)).astype(np.int32)
    x = datagen.student_t((M, d), 55 + M)
    w = asg.MLPWeights(W.to(DEV), None, L.AS_MLP_NEURON_SET)
    y, dbg = asg.as_sparse_swiglu_mlp(x.to(DEV), w, neuron_idx=torch.from_numpy(idx).to(DEV), debug=True)
    X = f64(x)
    h_ref = teal.silu(X @ Wg[idx].T) * (X @ Wu[idx].T)
    if n_act:
        assert rel_err(f64(dbg["h"])[:, :n_act], h_ref) < TOL
    ref = glass.neuron_set_mlp(X, Wg, Wu, Wd, idx)
    assert rel_err(y, ref) < TOL
    if n_act == 0:
        assert torch.count_nonzero(y).item() == 0


def test_neuron_set_full_equals_dense():
    announce("neuron-set full")
    d, f = 512, 2048
    W, Wg, Wu, Wd = _neuron_major(d, f, 3)
    x = datagen.student_t((1, d), 56)
    w = asg.MLPWeights(W.to(DEV), None, L.AS_MLP_NEURON_SET)
    y = asg.as_sparse_swiglu_mlp(x.to(DEV), w, flags=L.AS_FLAG_FORCE_DENSE)
    ref = glass.neuron_set_mlp(f64(x), Wg, Wu, Wd, np.arange(f))
    assert rel_err(y, ref) < TOL
    y2 = asg.as_sparse_swiglu_mlp(x.to(DEV), w, neuron_idx=torch.arange(f, dtype=torch.int32, device=DEV))
    assert rel_err(y2, ref) < TOL
