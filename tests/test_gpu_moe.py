"""GPU parity of the MoE router and the routed experts with intra-expert top-k,
checked stage by stage against the fp64 oracle (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import moe, teal, topk
from helpers import TOL, f64, rel_err, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
_W = {}


def _weights(E, d, f, fs):
    key = (E, d, f, fs)
    if key not in _W:
        _W.clear()
        w = datagen.moe_weights(5, 0, n_experts=E, d_model=d, d_ff_e=f, d_ff_shared=fs)
        dw = asg.MoEWeights(w["w_gate_up"].to(DEV), w["w_down"].to(DEV), w["w_router"].to(DEV),
                            asg.MLPWeights(w["s_gate_up"].to(DEV), w["s_down"].to(DEV)))
        _W[key] = (w, dw)
    return _W[key]


def _check_layer(E, d, f, fs, T, top, keep, seed, weights=None):
    w, dw = weights if weights is not None else _weights(E, d, f, fs)
    X = datagen.student_t((T, d), seed)
    Y, dbg = asg.moe_layer(X.to(DEV), dw, top, keep, debug=True)
    Xd = f64(X)
    Wr = f64(w["w_router"])
    # router: GPU logits within tolerance; selection and weights from the GPU's logits
    lg = f64(dbg["logits"])
    assert rel_err(lg, Xd @ Wr) < TOL
    ids = dbg["ids"].cpu().numpy()
    wts = f64(dbg["wts"])
    for t in range(T):
        sel = topk.value_topk(lg[t], top)
        order = sel[np.lexsort((sel, -lg[t][sel]))]
        assert ids[t].tolist() == order.tolist()
        z = lg[t][order]
        p = np.exp(z - z.max())
        np.testing.assert_allclose(wts[t], p / p.sum(), rtol=1e-5, atol=1e-7)
    # routed experts, stage by stage
    h = f64(dbg["h"])
    kp = dbg["keep"].cpu().numpy()
    sgu = f64(w["s_gate_up"])
    y_ref = np.zeros((T, d))
    for t in range(T):
        for j in range(top):
            e = int(ids[t, j])
            Wgu = f64(w["w_gate_up"][e])
            Wd = f64(w["w_down"][e])
            h_ref = teal.silu(Wgu[:, 0, :] @ Xd[t]) * (Wgu[:, 1, :] @ Xd[t])
            assert rel_err(h[t, j], h_ref) < TOL
            kidx = topk.value_topk(np.abs(h[t, j]), keep)            # exact on the GPU's h
            assert kp[t, j, :keep].tolist() == kidx.tolist()
            y_ref[t] += wts[t, j] * (h[t, j][kidx] @ Wd[kidx])
        y_ref[t] += teal.dense_mlp(Xd[t], sgu[:, 0, :], sgu[:, 1, :], f64(w["s_down"]))
    err = rel_err(Y, y_ref)
    assert err < TOL, err
    return ids


def test_moe_small_all_token_counts():
    for T in (1, 3, 8, 16):
        announce(f"moe small T={T}")
        _check_layer(8, 64, 48, 128, T, 2, 5, 100 + T)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_moe_workload(T):
    """128 experts, d_model 2048, d_ff_e 768, top-8 routing, keep the top 10% (77) of each
    routed expert's neurons, dense shared expert with d_ff 4096."""
    announce(f"moe workload T={T}")
    c = datagen.CFG5
    _check_layer(c["n_experts"], c["d_model"], c["d_ff_e"], c["d_ff_shared"], T, c["top"], c["keep"],
                 datagen.seed_for(5, T, "decode"))


def test_moe_keep_all_is_dense_moe():
    announce("moe keep-all")
    E, d, f, fs, T, top = 8, 64, 48, 128, 4, 2
    w, dw = _weights(E, d, f, fs)
    X = datagen.student_t((T, d), 7)
    Y = asg.moe_layer(X.to(DEV), dw, top, f)
    ref, _ = moe.moe_layer(f64(X), {k: f64(v) for k, v in w.items()}, top, f)
    assert rel_err(Y, ref) < TOL
    Y2 = asg.moe_layer(X.to(DEV), dw, top, 3, flags=L.AS_FLAG_FORCE_DENSE)
    assert rel_err(Y2, ref) < TOL


def test_moe_invalid_ids_and_determinism():
    announce("moe invalid ids")
    E, d, f, fs = 8, 64, 48, 128
    w, dw = _weights(E, d, f, fs)
    X = datagen.student_t((2, d), 8).to(DEV)
    ids = torch.tensor([[1, -1], [E, 3]], dtype=torch.int32, device=DEV)
    wts = torch.tensor([[0.5, 0.5], [0.25, 0.75]], dtype=torch.float32, device=DEV)
    Y, dbg = asg.as_sparse_moe_expert(X, dw, ids, wts, 5, debug=True)
    h = f64(dbg["h"])
    ref = np.zeros((2, d))
    for t, j, e, wt in ((0, 0, 1, 0.5), (1, 1, 3, 0.75)):
        kidx = topk.value_topk(np.abs(h[t, j]), 5)
        assert dbg["keep"][t, j].cpu().numpy().tolist() == kidx.tolist()
        ref[t] = wt * (h[t, j][kidx] @ f64(w["w_down"][e])[kidx])
    assert rel_err(Y, ref) < TOL
    assert dbg["keep"][0, 1].cpu().numpy().tolist() == [-1] * 5      # invalid expert: nothing kept
    Y2 = asg.as_sparse_moe_expert(X, dw, ids, wts, 5)
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("T,E,top", [(1, 128, 8), (3, 128, 8), (8, 128, 8), (2, 256, 6), (5, 512, 16), (1, 64, 64)])
def test_router_gemv_fused(T, E, top):
    """Logits GEMV and routing in one launch: the logits equal as_dense_gemv's (bit for
    bit up to 128 experts, the same plan), and the routing equals as_moe_router's on
    those logits, bit for bit."""
    announce(f"router gemv T={T} E={E} top={top}")
    d = 2048
    Wr = datagen.normal((d, E), 600 + E, std=0.02).to(DEV)
    X = datagen.student_t((T, d), 601 + T).to(DEV)
    logits, ids, wts = asg.as_moe_router_gemv(X, Wr, top)
    ref_logits = asg.as_dense_gemv(X, Wr)
    if E <= 128:
        assert torch.equal(logits, ref_logits)
    else:
        assert rel_err(logits, f64(ref_logits)) < 1e-5
    ids2, wts2 = asg.as_moe_router(logits, top)
    assert torch.equal(ids, ids2)
    assert torch.equal(wts, wts2)
    # against the oracle router on the same logits
    eye = np.eye(E)
    for t in range(T):
        ref_ids, ref_w, _ = moe.router(f64(logits[t]), eye, top)     # the oracle router on these logits
        assert ids[t].cpu().numpy().tolist() == ref_ids.tolist()
        assert rel_err(wts[t], ref_w) < 1e-5


@pytest.mark.parametrize("T", [1, 2, 4, 8])
@pytest.mark.parametrize("dense", [0, 1])
def test_moe_layer_one_stream_equals_composition(T, dense):
    """as_moe_layer (three launches on one stream, independent pieces side by side in
    one launch) gives the bits of the layer composed from the separate entry points
    (router GEMV with routing, dense shared MLP, routed experts accumulated) for every
    intermediate (logits, routing, h, keep sets); Y agrees to 1e-5 (the layer splits
    the shared expert's down stage one row range per CU and column tile, another
    fp32 summation order of the same terms)."""
    announce(f"moe one-stream T={T} dense={dense}")
    c = datagen.CFG5
    w, dw = _weights(c["n_experts"], c["d_model"], c["d_ff_e"], c["d_ff_shared"])
    X = datagen.student_t((T, c["d_model"]), datagen.seed_for(5, T, "decode")).to(DEV)
    flags = L.AS_FLAG_FORCE_DENSE if dense else 0
    assert asg.api.moe_layer_one_stream_ok(X, dw, c["top"], flags)
    Y1, d1 = asg.as_moe_layer(X, dw, c["top"], c["keep"], flags=flags, debug=True)
    Y2, d2 = asg.moe_layer(X, dw, c["top"], c["keep"], flags=flags, debug=True, one_stream=False)
    torch.cuda.synchronize()
    for k in ("logits", "ids", "wts", "h"):
        assert torch.equal(d1[k], d2[k]), k
    if not dense:
        assert torch.equal(d1["keep"], d2["keep"])
    assert rel_err(Y1, f64(Y2)) < 1e-5
    Y3 = asg.as_moe_layer(X, dw, c["top"], c["keep"], flags=flags)     # workspace reuse: the same bits
    assert torch.equal(Y3, Y1)


@pytest.mark.parametrize("T", [1, 4, 12])
def test_moe_atomic_splitk(T):
    """AS_FLAG_ATOMIC_SPLITK: each (token, slot) adds its weighted rows' sum into Y with
    atomics.  The layer (one stream up to 8 tokens, composed above) keeps the
    intermediates bit for bit and agrees with the deterministic layer to 1e-5 (same
    terms, another order of additions) and with the oracle; the routed experts alone
    overwrite a NaN-filled Y without AS_FLAG_ACCUMULATE and add onto it with it."""
    announce(f"moe atomic split-K T={T}")
    c = datagen.CFG5
    w, dw = _weights(c["n_experts"], c["d_model"], c["d_ff_e"], c["d_ff_shared"])
    X = datagen.student_t((T, c["d_model"]), datagen.seed_for(5, T, "decode")).to(DEV)
    Y1, d1 = asg.moe_layer(X, dw, c["top"], c["keep"], flags=L.AS_FLAG_ATOMIC_SPLITK, debug=True)
    Y2, d2 = asg.moe_layer(X, dw, c["top"], c["keep"], debug=True)
    torch.cuda.synchronize()
    for k in ("logits", "ids", "wts", "h", "keep"):
        assert torch.equal(d1[k], d2[k]), k
    assert rel_err(Y1, f64(Y2)) < 1e-5
    if T <= 4:
        _check_layer(c["n_experts"], c["d_model"], c["d_ff_e"], c["d_ff_shared"], T, c["top"], c["keep"],
                     datagen.seed_for(5, T, "decode"))
    Yn = torch.full((T, c["d_model"]), float("nan"), device=DEV)
    asg.as_sparse_moe_expert(X, dw, d2["ids"], d2["wts"], c["keep"], flags=L.AS_FLAG_ATOMIC_SPLITK, Y=Yn)
    Yr = asg.as_sparse_moe_expert(X, dw, d2["ids"], d2["wts"], c["keep"])
    assert rel_err(Yn, f64(Yr)) < 1e-5
    Y0 = torch.randn(T, c["d_model"], device=DEV)
    Ya = Y0.clone()
    asg.as_sparse_moe_expert(X, dw, d2["ids"], d2["wts"], c["keep"],
                             flags=L.AS_FLAG_ATOMIC_SPLITK | L.AS_FLAG_ACCUMULATE, Y=Ya)
    assert rel_err(Ya, f64(Y0) + f64(Yr)) < 1e-5


def test_moe_layer_one_stream_small_shapes():
    """Odd shapes through the one-stream layer against the oracle (E = 8, d_model 64,
    d_ff_e 48, shared d_ff 128; unaligned token rows take the LDS staging path)."""
    E, d, f, fs = 8, 64, 48, 128
    w, dw = _weights(E, d, f, fs)
    for T, top, keep in ((1, 2, 5), (3, 3, 1), (8, 8, 48), (5, 1, 0)):
        announce(f"moe one-stream small T={T} top={top} keep={keep}")
        X = datagen.student_t((T, d), 300 + T)
        assert asg.api.moe_layer_one_stream_ok(X.to(DEV), dw, top)
        Y, dbg = asg.as_moe_layer(X.to(DEV), dw, top, keep, debug=True)
        ref, _ = moe.moe_layer(f64(X), {k: f64(v) for k, v in w.items()}, top, keep)
        # the oracle's own routing and keep sets could differ from the GPU's on a near
        # tie; these seeds have none, so the whole layer is compared
        assert rel_err(Y, ref) < TOL
        # unaligned rows (one-element offset into a larger buffer)
        Xb = torch.zeros((T * d + 1,), dtype=X.dtype)
        Xb[1:] = X.reshape(-1)
        Xu = Xb.to(DEV)[1:].view(T, d)
        Yu = asg.as_moe_layer(Xu, dw, top, keep)
        assert torch.equal(Yu, Y)


def _router_ref(lg_t, top):
    """Oracle routing of one token's logits: ids in (logit desc, index asc) order, NaN last."""
    v = lg_t.astype(np.float64)
    sel = topk.value_topk(v, top)
    nan = np.isnan(v[sel])
    return sel[np.lexsort((sel, np.where(nan, 0.0, -v[sel]), nan))]


@pytest.mark.parametrize("E,top", [(128, 8), (256, 64), (512, 16), (1024, 8), (8, 8), (100, 7), (960, 33)])
def test_router_ties_and_special_values(E, top):
    """Exact routing (register top-k of the router) under heavy ties, +-0, NaN and
    infinities: ids equal the oracle's selection and order; weights where finite."""
    announce(f"router ties E={E} top={top}")
    rng = np.random.default_rng(E * 100 + top)
    T = 7
    lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)              # few values: ties
    lg[1] = 0.0
    lg[1, ::3] = -0.0                                                     # all equal, both zeros
    lg[2] = rng.standard_normal(E).astype(np.float32)
    lg[2, min(5, E - 1)] = np.nan
    lg[2, min(6, E - 1)] = np.inf
    lg[2, min(3, E - 1)] = -np.inf
    lg[3] = -np.inf
    lg[3, E // 2] = np.nan                                                # NaN ranks below -inf
    lg[4] = 1.0
    lg[4, E - 1] = np.nextafter(np.float32(1.0), np.float32(2.0))
    lg[5] = rng.standard_normal(E).astype(np.float32)
    lg[6] = np.round(rng.standard_normal(E) * 4).astype(np.float32) / 4
    ids, wts = asg.as_moe_router(torch.from_numpy(lg).to(DEV), top)
    ids = ids.cpu().numpy()
    wts = f64(wts)
    for t in range(T):
        ref = _router_ref(lg[t], top)
        assert ids[t].tolist() == ref.tolist(), t
        z = lg[t][ref].astype(np.float64)
        if np.all(np.isfinite(z)):
            p = np.exp(z - z.max())
            np.testing.assert_allclose(wts[t], p / p.sum(), rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("f,keep", [(300, 37), (768, 77), (1024, 500), (1100, 90)])
def test_expert_keep_sets_under_ties(f, keep):
    """Routed experts whose neurons repeat in a period of 5 (and every 7th neuron all
    zero, giving h = +-0): massive ties in |h|, which the keep sets must break toward
    the smaller neuron index, exactly as the oracle's top-k on the GPU's h."""
    announce(f"expert ties f={f} keep={keep}")
    E, d, T, top = 8, 64, 3, 2
    w = datagen.moe_weights(5, 9, n_experts=E, d_model=d, d_ff_e=f, d_ff_shared=128)
    gu = w["w_gate_up"].clone()
    gu[:, :, :, :] = gu[:, torch.arange(f) % 5, :, :]
    gu[:, ::7, :, :] = 0
    dw = asg.MoEWeights(gu.to(DEV), w["w_down"].to(DEV), w["w_router"].to(DEV),
                        asg.MLPWeights(w["s_gate_up"].to(DEV), w["s_down"].to(DEV)))
    X = datagen.student_t((T, d), 77).to(DEV)
    ids = torch.tensor([[0, 3], [3, 5], [7, 0]], dtype=torch.int32, device=DEV)
    wts = torch.tensor([[0.6, 0.4], [0.5, 0.5], [0.9, 0.1]], dtype=torch.float32, device=DEV)
    Y, dbg = asg.as_sparse_moe_expert(X, dw, ids, wts, keep, debug=True)
    h = f64(dbg["h"])
    kp = dbg["keep"].cpu().numpy()
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(top):
            e = int(ids[t, j])
            kidx = topk.value_topk(np.abs(h[t, j]), keep)
            assert kp[t, j, :keep].tolist() == kidx.tolist(), (t, j)
            ref[t] += float(wts[t, j]) * (h[t, j][kidx] @ f64(w["w_down"][e])[kidx])
    assert rel_err(Y, ref) < TOL


def test_moe_layer_fp16_and_composed_paths():
    """fp16 weights (outside the one-stream layer's bf16 instantiations) and 12 tokens
    (above its 8) take the composed path; both still match the oracle layer, and the
    binding reports which path a call takes."""
    E, d, f, fs = 16, 256, 96, 256
    w = datagen.moe_weights(5, 11, n_experts=E, d_model=d, d_ff_e=f, d_ff_shared=fs, dtype="f16")
    dw = asg.MoEWeights(w["w_gate_up"].to(DEV), w["w_down"].to(DEV), w["w_router"].to(DEV),
                        asg.MLPWeights(w["s_gate_up"].to(DEV), w["s_down"].to(DEV)))
    wb = datagen.moe_weights(5, 11, n_experts=E, d_model=d, d_ff_e=f, d_ff_shared=fs)
    dwb = asg.MoEWeights(wb["w_gate_up"].to(DEV), wb["w_down"].to(DEV), wb["w_router"].to(DEV),
                         asg.MLPWeights(wb["s_gate_up"].to(DEV), wb["s_down"].to(DEV)))
    for T, ww, src, one in ((3, dw, w, False), (12, dwb, wb, False), (3, dwb, wb, True)):
        announce(f"moe paths T={T} one_stream={one}")
        X = datagen.student_t((T, d), 500 + T)
        assert asg.api.moe_layer_one_stream_ok(X.to(DEV), ww, 4) == one
        # stage by stage against the oracle (selections on the GPU's logits and h)
        _check_layer(E, d, f, fs, T, 4, 20, 500 + T, weights=(src, ww))


@pytest.mark.parametrize("T", [1, 3])
def test_keep_sets_chosen_in_either_stage(T):
    """The keep sets are chosen at the end of the gate/up stage (the one-stream layer
    with more than 8 (token, slot) items: its last neuron block of each expert) or at
    the start of the down stage (the routed-expert entry point; the layer with at most
    8 items): the same selection on the same h gives the same bits either way."""
    announce(f"moe selection placement T={T}")
    c = datagen.CFG5
    w, dw = _weights(c["n_experts"], c["d_model"], c["d_ff_e"], c["d_ff_shared"])
    X = datagen.student_t((T, c["d_model"]), 900 + T).to(DEV)
    logits, ids, wts = asg.as_moe_router_gemv(X, dw.w_router, c["top"])
    Ye, de = asg.as_sparse_moe_expert(X, dw, ids, wts, c["keep"], debug=True)
    Yl, dl = asg.as_moe_layer(X, dw, c["top"], c["keep"], debug=True)
    torch.cuda.synchronize()
    assert torch.equal(dl["ids"], ids) and torch.equal(dl["wts"], wts)
    assert torch.equal(de["h"], dl["h"])
    assert torch.equal(de["keep"], dl["keep"])
