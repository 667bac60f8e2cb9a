"""GPU parity of the decoder-block glue (RMSNorm, GQA decode attention) and of a
thresholded Llama-3-8B-shaped decoder block, stage by stage (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import block, teal
from helpers import TOL, f64, rel_err, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_rmsnorm():
    announce("rmsnorm")
    for d, dt in ((4096, "bf16"), (777, "f32"), (64, "f16")):
        x = datagen.student_t((3, d), d, dtype=dt)
        y, c = asg.as_rmsnorm(x.to(DEV), copy=True)
        assert rel_err(y, block.rmsnorm(f64(x))) < 1e-5
        assert np.array_equal(f64(c), f64(x))


@pytest.mark.parametrize("n_ctx,n_q,n_kv,hd", [(2048, 32, 8, 128), (0, 4, 2, 128), (1, 8, 8, 128),
                                               (300, 16, 2, 128), (5000, 32, 8, 128), (70, 8, 1, 128),
                                               (5000, 8, 1, 128), (2100, 16, 2, 128)])
def test_attention(n_ctx, n_q, n_kv, hd):
    """Decode attention against the fp64 oracle; the shapes cover 1 to 64 key chunks per kv
    head (64 with one kv head and 5001 keys; 33 with two and 2101) and groups of 1 to 8."""
    announce(f"attention n_ctx={n_ctx}")
    rng = np.random.default_rng(n_ctx + n_q)
    q = torch.from_numpy(rng.standard_normal((n_q, hd)).astype(np.float32))
    kn = torch.from_numpy(rng.standard_normal((n_kv, hd)).astype(np.float32))
    vn = torch.from_numpy(rng.standard_normal((n_kv, hd)).astype(np.float32))
    kc, vc = datagen.kv_cache(3, n_ctx % 97, n_ctx=n_ctx, n_kv=n_kv, head_dim=hd)
    o = asg.as_gqa_decode_attention(q.to(DEV), kn.to(DEV), vn.to(DEV), kc.to(DEV), vc.to(DEV))
    ref = block.gqa_decode_attention(f64(q), f64(kc), f64(vc), f64(kn), f64(vn)).reshape(n_q, hd)
    assert rel_err(o, ref) < 1e-4
    # q = 0: equal scores -> the mean of the group's values
    o0 = asg.as_gqa_decode_attention(torch.zeros_like(q).to(DEV), kn.to(DEV), vn.to(DEV), kc.to(DEV), vc.to(DEV))
    Vall = np.concatenate([f64(vc), f64(vn)[None]], 0)
    assert rel_err(o0[0], Vall[:, 0].mean(0)) < 1e-5


_BLK = {}


def _block(layer):
    if layer not in _BLK:
        _BLK.clear()
        wqkv, wo = datagen.attn_weights(3, layer)
        wgu, wd = datagen.mlp_weights_input_major(3, layer, datagen.CFG2)
        kc, vc = datagen.kv_cache(3, layer)
        dev = asg.BlockWeights(wqkv.to(DEV), wo.to(DEV), asg.MLPWeights(wgu.to(DEV), wd.to(DEV)))
        _BLK[layer] = dict(wqkv=f64(wqkv), wo=f64(wo), wgu=f64(wgu), wd=f64(wd), kc=f64(kc), vc=f64(vc),
                           kcd=kc.to(DEV), vcd=vc.to(DEV), dev=dev)
    return _BLK[layer]


def _thresholds(b, calib, s):
    """Per-input thresholds at sparsity s from calibration vectors passed through the
    oracle block (sequential: each pool is taken with the upstream thresholds applied)."""
    t = dict(qkv=-np.inf, o=-np.inf, gu=-np.inf, d=-np.inf)
    keys = (("qkv", "xn"), ("o", "o"), ("gu", "xn2"), ("d", "h"))
    for k, pool_key in keys:
        pool = [block.decoder_block(x, b["wqkv"], b["wo"], b["wgu"], b["wd"], b["kc"], b["vc"], t)[pool_key]
                for x in calib]
        t[k] = teal.calibrate_threshold(np.array(pool), s)
    return t


@pytest.mark.parametrize("layer,fuse", [(0, 1), (31, 1), (0, 0)])
def test_decoder_block_stagewise(layer, fuse, monkeypatch):
    """Llama-3-8B-shaped block (q/o 4096x4096, k/v 4096x1024, MLP 4096->14336, 32/8 heads,
    2048 cached tokens) at the depth schedule's sparsity for this layer; with the RMS
    normalisations and residual adds folded into the projections (fuse=1, the
    default) and as separate launches (fuse=0)."""
    monkeypatch.setenv("AS_BLOCK_FUSE", str(fuse))
    s = datagen.cfg3_sparsity(layer)
    announce(f"block layer={layer} s={s:.2f}")
    b = _block(layer)
    calib = f64(datagen.student_t((16, 4096), datagen.seed_for(3, layer, "calib")))
    t = _thresholds(b, calib, s)
    tt = dict(qkv=t["qkv"], o=t["o"], gate_up=t["gu"], down=t["d"])
    x = datagen.student_t((4096,), datagen.seed_for(3, layer, "decode"))
    Y, g = asg.as_decoder_block(x.to(DEV), b["dev"], b["kcd"], b["vcd"], tt, debug=True)
    X = f64(x)
    G = {k: f64(v) for k, v in g.items()}
    assert rel_err(G["xn"], block.rmsnorm(X)) < 1e-5
    assert rel_err(G["qkv"], teal.masked_gemv(G["xn"], b["wqkv"], t["qkv"])) < TOL
    nq = 32 * 128
    q = G["qkv"][:nq].reshape(32, 128)
    kn = G["qkv"][nq:nq + 1024].reshape(8, 128)
    vn = G["qkv"][nq + 1024:].reshape(8, 128)
    assert rel_err(G["o"], block.gqa_decode_attention(q, b["kc"], b["vc"], kn, vn)) < TOL
    assert rel_err(G["h1"], X + teal.masked_gemv(G["o"], b["wo"], t["o"])) < TOL
    assert rel_err(G["xn2"], block.rmsnorm(G["h1"])) < 1e-5
    r = teal.swiglu_mlp_threshold(G["xn2"], b["wgu"][:, 0, :], b["wgu"][:, 1, :], b["wd"], t["gu"], t["d"])
    assert rel_err(G["h"], r["h"]) < TOL
    assert rel_err(Y, G["h1"] + teal.down_stage(G["h"], b["wd"], t["d"])) < TOL
    # end to end against the pure fp64 chain (information; asserted only without mask flips)
    ref = block.decoder_block(X, b["wqkv"], b["wo"], b["wgu"], b["wd"], b["kc"], b["vc"], t)
    print("e2e rel err", rel_err(Y, ref["out"]), flush=True)


@pytest.mark.parametrize("fuse", [1, 0])
def test_decoder_block_dense(fuse, monkeypatch):
    monkeypatch.setenv("AS_BLOCK_FUSE", str(fuse))
    announce(f"block dense fuse={fuse}")
    b = _block(0)
    x = datagen.student_t((4096,), 12345)
    tt = dict(qkv=9.0, o=9.0, gate_up=9.0, down=9.0)
    Y = asg.as_decoder_block(x.to(DEV), b["dev"], b["kcd"], b["vcd"], tt, flags=L.AS_FLAG_FORCE_DENSE)
    inf = dict(qkv=-np.inf, o=-np.inf, gu=-np.inf, d=-np.inf)
    ref = block.decoder_block(f64(x), b["wqkv"], b["wo"], b["wgu"], b["wd"], b["kc"], b["vc"], inf)
    assert rel_err(Y, ref["out"]) < TOL
