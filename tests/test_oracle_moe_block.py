"""Pins for the MoE, static-neuron-set and decoder-block oracles (CPU only)."""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import teal, topk, moe, block, glass
from activation_sparse_gemv_amd import datagen


def _f64(t):
    return t.to(torch.float64).numpy()


def _small_moe(E=8, d=64, fe=48, fs=96, seed=500):
    w = datagen.moe_weights(cfg=99, layer=seed % 97, n_experts=E, d_model=d, d_ff_e=fe, d_ff_shared=fs)
    return {k: _f64(v) for k, v in w.items()}


def _torch_swiglu(x, Wg, Wu, Wd):
    x, Wg, Wu, Wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, Wg, Wu, Wd))
    return ((F.silu(x @ Wg) * (x @ Wu)) @ Wd).numpy()


def test_router_brute_force_and_softmax():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(16)
    Wr = np.round(rng.standard_normal((16, 10)), 1)
    ids, wts, logits = moe.router(x, Wr, 3)
    # brute force over all 3-subsets: the selected set maximises the sorted logits, ties by index
    best = max(itertools.combinations(range(10), 3),
               key=lambda S: (sorted(logits[list(S)], reverse=True), [-i for i in S]))
    assert sorted(ids.tolist()) == sorted(best)
    # renormalised softmax over the selection == full softmax restricted and renormalised
    p = torch.softmax(torch.from_numpy(logits), 0).numpy()[ids]
    np.testing.assert_allclose(wts, p / p.sum(), rtol=1e-12)
    assert np.all(np.diff(logits[ids]) <= 0)


def test_expert_keep_all_is_dense_swiglu():
    w = _small_moe()
    x = _f64(datagen.student_t((64,), 7))
    e = 3
    y, h, kidx = moe.expert_sparse(x, w["w_gate_up"][e], w["w_down"][e], 48)
    ref = _torch_swiglu(x, w["w_gate_up"][e][:, 0, :].T, w["w_gate_up"][e][:, 1, :].T, w["w_down"][e])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)
    assert kidx.tolist() == list(range(48))


def test_expert_keep_k_is_top_magnitude():
    w = _small_moe()
    x = _f64(datagen.student_t((64,), 8))
    y, h, kidx = moe.expert_sparse(x, w["w_gate_up"][1], w["w_down"][1], 5)
    a = np.abs(h)
    assert a[kidx].min() >= np.delete(a, kidx).max()
    np.testing.assert_allclose(y, h[kidx] @ w["w_down"][1][kidx], rtol=1e-12)


def test_moe_layer_dense_special_case():
    """keep = d_ff_e gives the textbook dense MoE: softmax-weighted routed SwiGLUs + shared."""
    w = _small_moe()
    X = _f64(datagen.student_t((3, 64), 9))
    out, info = moe.moe_layer(X, w, top=2, keep=48)
    for t in range(3):
        logits = X[t] @ w["w_router"]
        sel = np.argsort(-logits, kind="stable")[:2]
        p = np.exp(logits[sel] - logits[sel].max())
        p /= p.sum()
        ref = sum(p[j] * _torch_swiglu(X[t], w["w_gate_up"][e][:, 0, :].T, w["w_gate_up"][e][:, 1, :].T,
                                       w["w_down"][e]) for j, e in enumerate(sel))
        ref = ref + _torch_swiglu(X[t], w["s_gate_up"][:, 0, :], w["s_gate_up"][:, 1, :], w["s_down"])
        np.testing.assert_allclose(out[t], ref, rtol=1e-11, atol=1e-14)


def test_moe_single_expert_weight_one():
    w = _small_moe(E=1)
    w["s_down"] = np.zeros_like(w["s_down"])     # silence the shared expert
    x = _f64(datagen.student_t((1, 64), 10))
    out, info = moe.moe_layer(x, w, top=1, keep=48)
    assert info[0]["weights"].tolist() == [1.0]
    ref = _torch_swiglu(x[0], w["w_gate_up"][0][:, 0, :].T, w["w_gate_up"][0][:, 1, :].T, w["w_down"][0])
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ gate-score experts
def test_expert_gate_score_hand_values():
    """d_model 2, three neurons, values worked by hand: g = (2, 0, -3); silu(2) =
    2/(1+e^-2) = 1.7616, silu(0) = 0, silu(-3) = -3/(1+e^3) = -0.1423; t = 0.1 keeps
    neurons 0 and 2; u = (1, -, 0.5); y = 1.7616 * 1 * Wd[0] - 0.1423 * 0.5 * Wd[2]."""
    x = np.array([1.0, 2.0])
    Wgu = np.array([[[2.0, 0.0], [1.0, 0.0]],
                    [[0.0, 0.0], [9.0, 9.0]],
                    [[-1.0, -1.0], [0.5, 0.0]]])
    Wd = np.array([[1.0, 0.0], [5.0, 5.0], [0.0, 2.0]])
    y, h, a, kidx = moe.expert_gate_score(x, Wgu, Wd, 0.1)
    s2, s3 = 2.0 / (1.0 + np.exp(-2.0)), -3.0 / (1.0 + np.exp(3.0))
    assert kidx.tolist() == [0, 2]
    np.testing.assert_allclose(a, [s2, 0.0, s3], rtol=1e-15)
    np.testing.assert_allclose(h, [s2, 0.0, 0.5 * s3], rtol=1e-15)
    np.testing.assert_allclose(y, [s2, 2.0 * 0.5 * s3], rtol=1e-15)
    # t between |silu(-3)| and silu(2) keeps neuron 0 only
    y1, _, _, k1 = moe.expert_gate_score(x, Wgu, Wd, 0.5)
    assert k1.tolist() == [0] and np.allclose(y1, [s2, 0.0], rtol=1e-15)


def test_expert_gate_score_limits_and_pruned_rows():
    """t = -inf is the dense SwiGLU expert; t = +inf drops every neuron (y = 0);
    at a median t the output equals the dense SwiGLU with the dropped neurons' up
    and down rows zeroed (the gate row is not pruned), and the kept set is exactly
    the neurons whose |silu(g)| exceeds t."""
    w = _small_moe()
    x = _f64(datagen.student_t((64,), 17))
    e = 5
    Wgu, Wd = w["w_gate_up"][e], w["w_down"][e]
    ref = _torch_swiglu(x, Wgu[:, 0, :].T, Wgu[:, 1, :].T, Wd)
    y, h, a, kidx = moe.expert_gate_score(x, Wgu, Wd, float("-inf"))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)
    assert kidx.tolist() == list(range(48))
    y, h, a, kidx = moe.expert_gate_score(x, Wgu, Wd, float("inf"))
    assert kidx.size == 0 and np.all(h == 0) and np.all(y == 0)
    g = torch.from_numpy(Wgu[:, 0, :] @ x)
    act = F.silu(g).numpy()
    t = float(np.float32(np.median(np.abs(act))))
    y, h, a, kidx = moe.expert_gate_score(x, Wgu, Wd, t)
    m = np.abs(act) > t
    assert kidx.tolist() == np.flatnonzero(m).tolist()
    Wu0, Wd0 = Wgu[:, 1, :].copy(), Wd.copy()
    Wu0[~m] = 0.0
    Wd0[~m] = 0.0
    np.testing.assert_allclose(y, _torch_swiglu(x, Wgu[:, 0, :].T, Wu0.T, Wd0), rtol=1e-11, atol=1e-15)


def test_moe_layer_gate_score_dense_limit_and_shared_only():
    """t = -inf equals the dense MoE layer (keep = d_ff_e); t = +inf leaves the
    shared expert alone; routing is the same as the top-k layer's."""
    w = _small_moe()
    X = _f64(datagen.student_t((3, 64), 19))
    out_d, info_d = moe.moe_layer(X, w, top=2, keep=48)
    out_g, info_g = moe.moe_layer_gate_score(X, w, top=2, t=float("-inf"))
    np.testing.assert_allclose(out_g, out_d, rtol=1e-12, atol=1e-15)
    for a, b in zip(info_d, info_g):
        assert a["ids"].tolist() == b["ids"].tolist()
    out_s, _ = moe.moe_layer_gate_score(X, w, top=2, t=float("inf"))
    for i in range(3):
        ref = _torch_swiglu(X[i], w["s_gate_up"][:, 0, :], w["s_gate_up"][:, 1, :], w["s_down"])
        np.testing.assert_allclose(out_s[i], ref, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ static neuron set
def test_neuron_set_full_is_dense_and_subset_is_masked():
    d, f = 64, 96
    W = _f64(datagen.mlp_weights_neuron_major(98, 1, d, f))
    Wg, Wu, Wd = W[:, 0], W[:, 1], W[:, 2]
    x = _f64(datagen.student_t((d,), 11))
    y = glass.neuron_set_mlp(x, Wg, Wu, Wd, np.arange(f))
    np.testing.assert_allclose(y, _torch_swiglu(x, Wg.T, Wu.T, Wd), rtol=1e-12, atol=1e-15)
    idx = np.array([3, 10, 50, 95])
    ys = glass.neuron_set_mlp(x, Wg, Wu, Wd, idx)
    h = teal.silu(Wg @ x) * (Wu @ x)
    m = topk.mask_from_index(idx, f)
    np.testing.assert_allclose(ys, np.where(m, h, 0) @ Wd, rtol=1e-12, atol=1e-16)


def test_local_signal():
    h = np.array([[1.0, -2.0, 0.0], [-3.0, 2.0, 0.5]])
    assert glass.local_signal(h).tolist() == [2.0, 2.0, 0.25]
    W = _f64(datagen.mlp_weights_neuron_major(98, 2, 32, 40))
    X = _f64(datagen.student_t((5, 32), 12))
    hp = glass.prompt_h(X, W[:, 0], W[:, 1])
    ref = F.silu(torch.from_numpy(X) @ torch.from_numpy(W[:, 0]).T) * (torch.from_numpy(X) @ torch.from_numpy(W[:, 1]).T)
    np.testing.assert_allclose(hp, ref.numpy(), rtol=1e-12, atol=1e-16)


# ------------------------------------------------------------ decoder block
def test_rmsnorm_matches_torch():
    x = _f64(datagen.student_t((4, 256), 13))
    ref = F.rms_norm(torch.from_numpy(x), (256,), eps=1e-5).numpy()
    np.testing.assert_allclose(block.rmsnorm(x), ref, rtol=1e-12)


def test_attention_closed_forms_and_sdpa():
    n_q, n_kv, hd, n = 8, 2, 16, 33
    rng = np.random.default_rng(14)
    q = rng.standard_normal((n_q, hd))
    K = rng.standard_normal((n, n_kv, hd))
    V = rng.standard_normal((n, n_kv, hd))
    kn, vn = rng.standard_normal((n_kv, hd)), rng.standard_normal((n_kv, hd))
    o = block.gqa_decode_attention(q, K, V, kn, vn).reshape(n_q, hd)
    # against torch SDPA (fp64, CPU) with KV heads repeated per query group
    Kall = np.concatenate([K, kn[None]], 0)
    Vall = np.concatenate([V, vn[None]], 0)
    kt = torch.from_numpy(Kall).permute(1, 0, 2).repeat_interleave(n_q // n_kv, 0)
    vt = torch.from_numpy(Vall).permute(1, 0, 2).repeat_interleave(n_q // n_kv, 0)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], kt, vt)[:, 0, :].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-13)
    # equal scores (q = 0) -> the mean of V over all keys of the head's group
    o0 = block.gqa_decode_attention(np.zeros((n_q, hd)), K, V, kn, vn).reshape(n_q, hd)
    np.testing.assert_allclose(o0[0], Vall[:, 0].mean(0), rtol=1e-12)
    np.testing.assert_allclose(o0[n_q - 1], Vall[:, n_kv - 1].mean(0), rtol=1e-12)
    # no cached keys -> the new value itself
    o1 = block.gqa_decode_attention(q, K[:0], V[:0], kn, vn).reshape(n_q, hd)
    np.testing.assert_allclose(o1[5], vn[5 // (n_q // n_kv)], rtol=1e-14)


def test_decoder_block_dense_special_case():
    d, nq, nkv, hd, f, n = 64, 4, 2, 16, 96, 10
    rng = np.random.default_rng(15)
    wqkv = rng.standard_normal((d, (nq + 2 * nkv) * hd)) * 0.1
    wo = rng.standard_normal((nq * hd, d)) * 0.1
    wgu = rng.standard_normal((d, 2, f)) * 0.1
    wd = rng.standard_normal((f, d)) * 0.1
    K, V = rng.standard_normal((n, nkv, hd)), rng.standard_normal((n, nkv, hd))
    x = rng.standard_normal(d)
    inf = dict(qkv=-np.inf, o=-np.inf, gu=-np.inf, d=-np.inf)
    r = block.decoder_block(x, wqkv, wo, wgu, wd, K, V, inf, nq, nkv, hd)
    # independent composition in torch fp64
    xt = torch.from_numpy(x)
    xn = F.rms_norm(xt, (d,), eps=1e-5)
    qkv = xn @ torch.from_numpy(wqkv)
    q = qkv[: nq * hd].reshape(nq, 1, hd)
    kk = torch.cat([torch.from_numpy(K), qkv[nq * hd:(nq + nkv) * hd].reshape(1, nkv, hd)], 0)
    vv = torch.cat([torch.from_numpy(V), qkv[(nq + nkv) * hd:].reshape(1, nkv, hd)], 0)
    kk = kk.permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
    vv = vv.permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
    o = F.scaled_dot_product_attention(q, kk, vv).reshape(-1)
    h1 = xt + o @ torch.from_numpy(wo)
    xn2 = F.rms_norm(h1, (d,), eps=1e-5)
    W = torch.from_numpy(wgu)
    out = h1 + (F.silu(xn2 @ W[:, 0]) * (xn2 @ W[:, 1])) @ torch.from_numpy(wd)
    np.testing.assert_allclose(r["out"], out.numpy(), rtol=1e-11, atol=1e-13)
    # thresholds on: the o-proj input mask is applied as written
    t = dict(qkv=np.float32(0.5), o=np.float32(0.3), gu=np.float32(0.5), d=np.float32(0.01))
    r2 = block.decoder_block(x, wqkv, wo, wgu, wd, K, V, t, nq, nkv, hd)
    np.testing.assert_allclose(r2["y_att"], teal.masked_gemv(r2["o"], wo, t["o"]), rtol=1e-13)


def test_decoder_block_rows_are_independent_tokens():
    """Tokens passed together [T, d] give row by row the results of one-token calls
    (the rows only share the matrix products), with thresholds on."""
    d, nq, nkv, hd, f, n = 64, 4, 2, 16, 96, 10
    rng = np.random.default_rng(16)
    wqkv = rng.standard_normal((d, (nq + 2 * nkv) * hd)) * 0.1
    wo = rng.standard_normal((nq * hd, d)) * 0.1
    wgu = rng.standard_normal((d, 2, f)) * 0.1
    wd = rng.standard_normal((f, d)) * 0.1
    K, V = rng.standard_normal((n, nkv, hd)), rng.standard_normal((n, nkv, hd))
    X = rng.standard_normal((3, d))
    t = dict(qkv=np.float32(0.5), o=np.float32(0.3), gu=np.float32(0.5), d=np.float32(0.01))
    rb = block.decoder_block(X, wqkv, wo, wgu, wd, K, V, t, nq, nkv, hd)
    for i in range(3):
        r1 = block.decoder_block(X[i], wqkv, wo, wgu, wd, K, V, t, nq, nkv, hd)
        for k in ("xn", "qkv", "o", "h1", "xn2", "h", "out"):
            np.testing.assert_allclose(rb[k][i], r1[k], rtol=1e-13, atol=1e-15, err_msg=k)
