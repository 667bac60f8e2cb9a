"""GPU parity of the routed experts and the MoE layer under the gate-score keep rule
(|silu(g)| > t, up and down over the kept neurons), stage by stage against the fp64
oracle (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import moe, teal
from helpers import TOL, f64, rel_err, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_A = 1e-5     # silu(g): an fp32 dot product of d_model exact bf16/f16 products, then silu
TOL_Y = 2e-5     # the weighted down rows of the GPU's own h, fp32


def _experts(E, d, f, dt="bf16", seed_layer=0):
    w = datagen.moe_weights(5, seed_layer, n_experts=E, d_model=d, d_ff_e=f, d_ff_shared=64, dtype=dt)
    dw = asg.MoEWeights(w["w_gate_up"].to(DEV), w["w_down"].to(DEV))
    return w, dw


def _routing(T, top, E, seed, crowd=False):
    """Distinct experts per token (random, or all tokens on the same few experts to
    put many items on one expert) and positive weights."""
    rng = np.random.default_rng(seed)
    if crowd:
        ids = np.tile(np.arange(top), (T, 1))
    else:
        ids = np.stack([rng.choice(E, top, replace=False) for _ in range(T)])
    wts = rng.uniform(0.05, 1.0, (T, top))
    return torch.from_numpy(ids.astype(np.int32)), torch.from_numpy(wts.astype(np.float32))


def _check_expert(w, X, ids, wts, t, Y, dbg, accumulate_onto=None):
    """Every stage against the oracle fed the GPU's own upstream values."""
    T, top = ids.shape
    E = w["w_gate_up"].shape[0]
    Xd = f64(X)
    a, h = f64(dbg["a"]), f64(dbg["h"])
    y_ref = np.zeros_like(f64(Y)) if accumulate_onto is None else f64(accumulate_onto).copy()
    flips = 0
    e2e = np.zeros_like(y_ref)
    for i in range(T):
        for j in range(top):
            e = int(ids[i, j])
            if not 0 <= e < E:
                continue
            Wgu, Wd = f64(w["w_gate_up"][e]), f64(w["w_down"][e])
            ye, _, a_ref, kidx = moe.expert_gate_score(Xd[i], Wgu, Wd, t)
            assert rel_err(a[i, j], a_ref) < TOL_A
            keep = teal.magnitude_mask(a[i, j], t)             # exact on the GPU's a
            assert np.all(h[i, j][~keep] == 0.0)
            want = np.where(keep, a[i, j] * (Wgu[:, 1, :] @ Xd[i]), 0.0)
            assert rel_err(h[i, j], want) < TOL_A
            y_ref[i] += float(wts[i, j]) * (h[i, j] @ Wd)
            flips += int((keep != np.isin(np.arange(keep.size), kidx)).sum())
            e2e[i] += float(wts[i, j]) * ye
    assert rel_err(Y, y_ref) < TOL_Y
    if accumulate_onto is None and flips == 0:
        assert rel_err(Y, e2e) < 1e-4
    return flips


@pytest.mark.parametrize("E,d,f,T,top,crowd,xdt,dt", [
    (8, 64, 48, 1, 2, False, "bf16", "bf16"),        # registers, one token
    (8, 64, 48, 2, 2, True, "bf16", "bf16"),         # registers, two items on one expert
    (8, 64, 48, 7, 3, True, "f32", "f16"),           # LDS staging, groups of 4 and a ragged 3
    (16, 520, 300, 3, 4, False, "bf16", "bf16"),     # d_model not a multiple of 512
    (8, 2048, 1100, 5, 2, True, "f16", "bf16"),      # d_ff above 1024, LDS path
    (4, 64, 8192, 2, 2, False, "bf16", "bf16"),      # the largest expert row count
    (128, 2048, 768, 16, 8, False, "bf16", "bf16"),  # the 128-expert workload, 16 tokens
])
def test_gate_expert_stagewise(E, d, f, T, top, crowd, xdt, dt):
    announce(f"moe gate expert E={E} d={d} f={f} T={T} top={top} crowd={crowd} {xdt}/{dt}")
    w, dw = _experts(E, d, f, dt)
    X = datagen.student_t((T, d), 900 + T + d, dtype=xdt)
    ids, wts = _routing(T, top, E, 901 + T, crowd)
    # t at the median |silu(g)| of the routed neurons
    _, d0 = asg.as_sparse_moe_expert_gate(X.to(DEV), dw, ids.to(DEV), wts.to(DEV), float("-inf"), debug=True)
    t = float(np.float32(np.median(np.abs(f64(d0["a"])))))
    Y, dbg = asg.as_sparse_moe_expert_gate(X.to(DEV), dw, ids.to(DEV), wts.to(DEV), t, debug=True)
    flips = _check_expert(w, X, ids.numpy(), wts.numpy(), t, Y, dbg)
    print(f"t {t:.4g}, flips vs fp64 {flips}", flush=True)


def test_gate_expert_unaligned_input_and_invalid_ids():
    """Rows not 16-byte aligned (element loads); ids outside [0, E) contribute nothing."""
    E, d, f, T, top = 8, 72, 96, 3, 3
    w, dw = _experts(E, d, f)
    Xb = datagen.student_t((T * d + 1,), 31)
    X = Xb.to(DEV)[1:].view(T, d)
    ids = torch.tensor([[0, -1, 5], [E, 2, 3], [7, 6, -5]], dtype=torch.int32)
    wts = torch.tensor([[0.5, 0.9, 0.25], [0.3, 0.6, 0.1], [1.0, 0.2, 0.4]])
    Y, dbg = asg.as_sparse_moe_expert_gate(X, dw, ids.to(DEV), wts.to(DEV), 0.05, debug=True)
    _check_expert(w, X.cpu(), ids.numpy(), wts.numpy(), 0.05, Y, dbg)


def test_gate_expert_limits_and_accumulate():
    """t = -inf keeps every neuron and equals the top-k path with keep = d_ff_e (same
    h bits, same kept rows in the same order) and FORCE_DENSE; t = +inf gives Y = 0;
    ACCUMULATE adds onto Y; the atomic split-K flag agrees within fp32 reordering."""
    E, d, f, T, top = 16, 256, 200, 4, 4
    w, dw = _experts(E, d, f)
    X = datagen.student_t((T, d), 41).to(DEV)
    ids, wts = (v.to(DEV) for v in _routing(T, top, E, 42))
    y_all, dbg = asg.as_sparse_moe_expert_gate(X, dw, ids, wts, float("-inf"), debug=True)
    y_topk, dk = asg.as_sparse_moe_expert(X, dw, ids, wts, f, debug=True)
    assert torch.equal(dbg["h"], dk["h"])
    assert torch.count_nonzero(dbg["h"]).item() == dbg["h"].numel()
    assert torch.equal(y_all, y_topk)
    y_fd = asg.as_sparse_moe_expert_gate(X, dw, ids, wts, 0.3, flags=L.AS_FLAG_FORCE_DENSE)
    assert torch.equal(y_fd, y_all)
    y_none = asg.as_sparse_moe_expert_gate(X, dw, ids, wts, float("inf"))
    assert torch.count_nonzero(y_none).item() == 0
    base = datagen.student_t((T, d), 43).float().to(DEV)
    Y = base.clone()
    _, dbg = asg.as_sparse_moe_expert_gate(X, dw, ids, wts, 0.2, flags=L.AS_FLAG_ACCUMULATE, Y=Y, debug=True)
    _check_expert(w, X.cpu(), ids.cpu().numpy(), wts.cpu().numpy(), 0.2, Y, dbg, accumulate_onto=base)
    y_at = asg.as_sparse_moe_expert_gate(X, dw, ids, wts, 0.2, flags=L.AS_FLAG_ATOMIC_SPLITK)
    y_det = asg.as_sparse_moe_expert_gate(X, dw, ids, wts, 0.2)
    assert rel_err(y_at, y_det) < 1e-5
    assert torch.equal(y_det, asg.as_sparse_moe_expert_gate(X, dw, ids, wts, 0.2))
    with pytest.raises(L.ASError):
        asg.as_sparse_moe_expert_gate(X, dw, ids, wts, float("nan"))


_LW = {}


def _layer_weights():
    if not _LW:
        c = datagen.CFG5
        w = datagen.moe_weights(5, 0, n_experts=c["n_experts"], d_model=c["d_model"], d_ff_e=c["d_ff_e"],
                                d_ff_shared=c["d_ff_shared"])
        dw = asg.MoEWeights(w["w_gate_up"].to(DEV), w["w_down"].to(DEV), w["w_router"].to(DEV),
                            asg.MLPWeights(w["s_gate_up"].to(DEV), w["s_down"].to(DEV)))
        _LW["w"] = (w, dw)
    return _LW["w"]


@pytest.mark.parametrize("T", [1, 4, 8])
def test_gate_moe_layer_one_stream(T):
    """The 128-expert workload through the one-stream layer: routing equals the top-k
    layer's bit for bit, routed stages as for the expert entry, Y = dense shared
    expert + the weighted routed sum (normwise 2e-3); the composed path (separate
    entry points, shared expert on a second stream) agrees."""
    announce(f"moe gate layer T={T}")
    w, dw = _layer_weights()
    c = datagen.CFG5
    top = c["top"]
    X = datagen.student_t((T, c["d_model"]), 950 + T)
    Xg = X.to(DEV)
    _, d0 = asg.as_moe_layer_gate(Xg, dw, top, float("-inf"), debug=True)
    t = float(np.float32(np.quantile(np.abs(f64(d0["a"])), 0.85)))
    Y, dbg = asg.as_moe_layer_gate(Xg, dw, top, t, debug=True)
    _, dk = asg.as_moe_layer(Xg, dw, top, c["keep"], debug=True)
    assert torch.equal(dbg["ids"], dk["ids"]) and torch.equal(dbg["wts"], dk["wts"])
    ids, wts = dbg["ids"].cpu().numpy(), dbg["wts"].cpu().numpy()
    sgu = f64(w["s_gate_up"])
    shared = np.stack([teal.dense_mlp(f64(X)[i], sgu[:, 0, :], sgu[:, 1, :], f64(w["s_down"])) for i in range(T)])
    a, h = f64(dbg["a"]), f64(dbg["h"])
    y_ref = shared.copy()
    for i in range(T):
        for j in range(top):
            e = int(ids[i, j])
            Wgu, Wd = f64(w["w_gate_up"][e]), f64(w["w_down"][e])
            a_ref = teal.silu(Wgu[:, 0, :] @ f64(X)[i])
            assert rel_err(a[i, j], a_ref) < TOL_A
            keep = teal.magnitude_mask(a[i, j], t)
            assert np.all(h[i, j][~keep] == 0.0)
            assert rel_err(h[i, j], np.where(keep, a[i, j] * (Wgu[:, 1, :] @ f64(X)[i]), 0.0)) < TOL_A
            y_ref[i] += float(wts[i, j]) * (h[i, j] @ Wd)
    assert rel_err(Y, y_ref) < TOL
    Yc = asg.moe_layer(Xg, dw, top, 0, one_stream=False, t_gate=t)
    assert rel_err(Yc, Y) < 1e-4
    assert torch.equal(Y, asg.as_moe_layer_gate(Xg, dw, top, t))
