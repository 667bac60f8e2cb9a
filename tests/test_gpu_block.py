"""GPU parity of the decoder-block glue (RMSNorm, GQA decode attention), of a
thresholded Llama-3-8B-shaped decoder block stage by stage, and of the 32-block
chain with thresholds calibrated block to block (run on an MI355X).

Stage-wise parity: the GPU exports every tensor it thresholded (xn, o, xn2, h) and
the mask it applied; the oracle's mask of that tensor must equal the GPU's bit for
bit, and each stage's output must be within tolerance of the oracle fed the GPU's
inputs of that stage.  The pure fp64 chain is reported as information."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import block, teal
from helpers import TOL, f64, rel_err, bits_to_bool, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PLAIN = 2e-5     # stages that are plain GEMVs (fp32 accumulation)
TOL_H = 1e-5     # the SwiGLU intermediate h


def test_rmsnorm():
    announce("rmsnorm")
    for d, dt in ((4096, "bf16"), (777, "f32"), (64, "f16")):
        x = datagen.student_t((3, d), d, dtype=dt)
        y, c = asg.as_rmsnorm(x.to(DEV), copy=True)
        assert rel_err(y, block.rmsnorm(f64(x))) < 1e-5
        assert np.array_equal(f64(c), f64(x))


@pytest.mark.parametrize("n_ctx,n_q,n_kv,hd", [(2048, 32, 8, 128), (0, 4, 2, 128), (1, 8, 8, 128),
                                               (300, 16, 2, 128), (5000, 32, 8, 128), (70, 8, 1, 128),
                                               (5000, 8, 1, 128), (2100, 16, 2, 128), (4096, 64, 8, 128),
                                               (20000, 4, 4, 128), (9000, 32, 16, 128), (32767, 8, 8, 128)])
def test_attention(n_ctx, n_q, n_kv, hd):
    """Decode attention against the fp64 oracle; the shapes cover 1 to 256 key chunks per kv
    head, chunks of up to 64 and up to 128 cached keys (two and four row steps), groups of 1
    to 8 query heads per kv head in both chunk sizes, the longest context (32767), and a
    second call bit-identical to the first (the chunk merge runs in a fixed order)."""
    announce(f"attention n_ctx={n_ctx}")
    rng = np.random.default_rng(n_ctx + n_q)
    q = torch.from_numpy(rng.standard_normal((n_q, hd)).astype(np.float32))
    kn = torch.from_numpy(rng.standard_normal((n_kv, hd)).astype(np.float32))
    vn = torch.from_numpy(rng.standard_normal((n_kv, hd)).astype(np.float32))
    kc, vc = datagen.kv_cache(3, n_ctx % 97, n_ctx=n_ctx, n_kv=n_kv, head_dim=hd)
    o = asg.as_gqa_decode_attention(q.to(DEV), kn.to(DEV), vn.to(DEV), kc.to(DEV), vc.to(DEV))
    ref = block.gqa_decode_attention(f64(q), f64(kc), f64(vc), f64(kn), f64(vn)).reshape(n_q, hd)
    assert rel_err(o, ref) < 1e-4
    o2 = asg.as_gqa_decode_attention(q.to(DEV), kn.to(DEV), vn.to(DEV), kc.to(DEV), vc.to(DEV))
    assert torch.equal(o, o2)
    # q = 0: equal scores -> the mean of the group's values
    o0 = asg.as_gqa_decode_attention(torch.zeros_like(q).to(DEV), kn.to(DEV), vn.to(DEV), kc.to(DEV), vc.to(DEV))
    Vall = np.concatenate([f64(vc), f64(vn)[None]], 0)
    assert rel_err(o0[0], Vall[:, 0].mean(0)) < 1e-5


def _block_weights(layer):
    wqkv, wo = datagen.attn_weights(3, layer)
    wgu, wd = datagen.mlp_weights_input_major(3, layer, datagen.CFG2)
    kc, vc = datagen.kv_cache(3, layer)
    dev = asg.BlockWeights(wqkv.to(DEV), wo.to(DEV), asg.MLPWeights(wgu.to(DEV), wd.to(DEV)))
    host = dict(wqkv=f64(wqkv), wo=f64(wo), wgu=f64(wgu), wd=f64(wd), kc=f64(kc), vc=f64(vc))
    return host, dev, kc.to(DEV), vc.to(DEV)


_BLK = {}


def _block(layer):
    if layer not in _BLK:
        _BLK.clear()
        host, dev, kcd, vcd = _block_weights(layer)
        _BLK[layer] = dict(host, dev=dev, kcd=kcd, vcd=vcd)
    return _BLK[layer]


def _oracle_t(t):
    """as_decoder_block's threshold names -> the oracle block's."""
    return dict(qkv=t["qkv"], o=t["o"], gu=t["gate_up"], d=t["down"])


def _check_masks(G, t):
    """Each of the four thresholded inputs: the mask the GPU applied equals the
    oracle's mask of the tensor the GPU exported, bit for bit; nnz and the ascending
    index lists agree."""
    flips = {}
    for key, src, tk in (("qkv_in", "xn", "qkv"), ("o_in", "o", "o"), ("gate_up_in", "xn2", "gate_up"),
                         ("down_in", "h", "down")):
        v = f64(G[src])
        m = teal.magnitude_mask(v, t[tk])
        got = bits_to_bool(G[key]["bits"], v.size)[0]
        assert np.array_equal(got, m), (key, int((got != m).sum()))
        assert int(G[key]["nnz"][0]) == int(m.sum()), key
        if G[key].get("idx") is not None:
            assert np.array_equal(G[key]["idx"][0, :int(m.sum())].cpu().numpy(), np.flatnonzero(m)), key
        flips[key] = m
    return flips


def _check_values(gs, ys, xs, b, t):
    """Every stage of every token within tolerance of the oracle fed the GPU's inputs
    of that stage (tokens in one batch of oracle products, errors per token).
    gs: per-token debug dicts, ys: outputs, xs: [T, d] fp64 inputs."""
    o_t = _oracle_t(t)
    G = {k: np.stack([f64(g[k]) for g in gs]) for k in ("xn", "qkv", "o", "h1", "xn2", "h")}
    Y = np.stack([f64(y) for y in ys])

    def rows(got, ref, tol, what):
        for i in range(got.shape[0]):
            e = rel_err(got[i], ref[i])
            assert e < tol, (what, i, e)

    rows(G["xn"], block.rmsnorm(xs), 1e-5, "xn")
    rows(G["qkv"], teal.masked_gemv(G["xn"], b["wqkv"], o_t["qkv"]), PLAIN, "qkv")
    nq = 32 * 128
    for i in range(G["qkv"].shape[0]):
        q = G["qkv"][i, :nq].reshape(32, 128)
        kn = G["qkv"][i, nq:nq + 1024].reshape(8, 128)
        vn = G["qkv"][i, nq + 1024:].reshape(8, 128)
        assert rel_err(G["o"][i], block.gqa_decode_attention(q, b["kc"], b["vc"], kn, vn)) < 1e-4, ("o", i)
    rows(G["h1"], xs + teal.masked_gemv(G["o"], b["wo"], o_t["o"]), PLAIN, "h1")
    rows(G["xn2"], block.rmsnorm(G["h1"]), 1e-5, "xn2")
    r = teal.swiglu_mlp_threshold(G["xn2"], b["wgu"][:, 0, :], b["wgu"][:, 1, :], b["wd"], o_t["gu"], o_t["d"])
    rows(G["h"], r["h"], TOL_H, "h")
    rows(Y, G["h1"] + teal.down_stage(G["h"], b["wd"], o_t["d"]), PLAIN, "y")


def _thresholds(b, calib, s):
    """Per-input thresholds at sparsity s from calibration vectors passed through the
    oracle block (sequential: each pool is taken with the upstream thresholds applied)."""
    t = dict(qkv=-np.inf, o=-np.inf, gu=-np.inf, d=-np.inf)
    keys = (("qkv", "xn"), ("o", "o"), ("gu", "xn2"), ("d", "h"))
    for k, pool_key in keys:
        pool = block.decoder_block(calib, b["wqkv"], b["wo"], b["wgu"], b["wd"], b["kc"], b["vc"], t)[pool_key]
        t[k] = teal.calibrate_threshold(pool, s)
    return dict(qkv=t["qkv"], o=t["o"], gate_up=t["gu"], down=t["d"])


@pytest.mark.parametrize("layer,fuse", [(0, 1), (31, 1), (0, 0)])
def test_decoder_block_stagewise(layer, fuse):
    """Llama-3-8B-shaped block (q/o 4096x4096, k/v 4096x1024, MLP 4096->14336, 32/8 heads,
    2048 cached tokens) at the depth schedule's sparsity for this layer, 8 decode
    tokens; with the RMS normalisations and residual adds folded into the projections
    (the default) and as launches of their own (AS_FLAG_NO_FUSION)."""
    s = datagen.cfg3_sparsity(layer)
    announce(f"block layer={layer} s={s:.2f} fuse={fuse}")
    b = _block(layer)
    calib = f64(datagen.student_t((16, 4096), datagen.seed_for(3, layer, "calib")))
    t = _thresholds(b, calib, s)
    flags = 0 if fuse else L.AS_FLAG_NO_FUSION
    toks = datagen.student_t((8, 4096), datagen.seed_for(3, layer, "decode"))
    ref = block.decoder_block(f64(toks), b["wqkv"], b["wo"], b["wgu"], b["wd"], b["kc"], b["vc"], _oracle_t(t))
    ys, gs = [], []
    for i in range(8):
        Y, g = asg.as_decoder_block(toks[i].to(DEV), b["dev"], b["kcd"], b["vcd"], t, flags=flags, debug=True)
        masks = _check_masks(g, t)
        ys.append(Y)
        gs.append(g)
        # the pure fp64 chain: masks may flip where a value lies within rounding of t;
        # without a flip the end-to-end error is held to the tolerance
        nflip = sum(int((masks[k] != teal.magnitude_mask(ref[src][i], t[tk])).sum())
                    for k, src, tk in (("qkv_in", "xn", "qkv"), ("o_in", "o", "o"), ("gate_up_in", "xn2", "gate_up"),
                                       ("down_in", "h", "down")))
        e2e = rel_err(Y, ref["out"][i])
        print(f"token {i}: flips vs fp64 chain {nflip}, e2e rel err {e2e:.2e}", flush=True)
        if nflip == 0:
            assert e2e < TOL
    _check_values(gs, ys, f64(toks), b, t)


@pytest.mark.parametrize("fuse", [1, 0])
def test_decoder_block_dense(fuse):
    announce(f"block dense fuse={fuse}")
    b = _block(0)
    x = datagen.student_t((4096,), 12345)
    tt = dict(qkv=9.0, o=9.0, gate_up=9.0, down=9.0)
    flags = L.AS_FLAG_FORCE_DENSE | (0 if fuse else L.AS_FLAG_NO_FUSION)
    Y = asg.as_decoder_block(x.to(DEV), b["dev"], b["kcd"], b["vcd"], tt, flags=flags)
    inf = dict(qkv=-np.inf, o=-np.inf, gu=-np.inf, d=-np.inf)
    ref = block.decoder_block(f64(x), b["wqkv"], b["wo"], b["wgu"], b["wd"], b["kc"], b["vc"], inf)
    assert rel_err(Y, ref["out"]) < TOL


@pytest.mark.timeout(1200)
def test_block_chain_32_calibrated_block_to_block():
    """The 32-block Llama-3-8B-shaped chain with the 30% -> 60% depth schedule.

    Calibration: 256 Student-t(3) vectors enter block 0; each block's four pools are
    taken in order with the earlier thresholds applied and the block's outputs are
    the next block's calibration vectors; thresholds come from the library's
    calibration kernel and equal the oracle's nearest-rank threshold of the same
    pools bit for bit.  Parity: 8 decode tokens pass through all 32 blocks; at every
    block the four masks are bit-exact on the GPU's own tensors and every stage is
    within tolerance of the oracle fed the GPU's inputs.  The pure fp64 chain of the
    same tokens (with the same thresholds) is reported: mask flips per block and the
    Jaccard index of the down-input masks."""
    n_blocks = datagen.CFG3_ATTN["n_blocks"]
    xc = datagen.student_t((datagen.N_CALIB, 4096), datagen.seed_for(3, 0, "calib")).to(DEV)
    toks = datagen.student_t((8, 4096), datagen.seed_for(3, 0, "decode"))
    x_gpu = [toks[i].to(DEV) for i in range(8)]
    x_ref = f64(toks)
    tot_flips, jac = 0, []
    for layer in range(n_blocks):
        s = datagen.cfg3_sparsity(layer, n_blocks)
        host, dev, kcd, vcd = _block_weights(layer)
        t, y_cal, pools = asg.calibrate_decoder_block(xc, dev, kcd, vcd, s, keep_pools=True)
        for k, pool in pools.items():
            ref_t = teal.calibrate_threshold(f64(pool), s)
            assert np.float32(t[k]).tobytes() == np.float32(ref_t).tobytes(), (layer, k, t[k], ref_t)
        outs, dbgs, gs = [], [], []
        for i in range(8):
            Y, g = asg.as_decoder_block(x_gpu[i], dev, kcd, vcd, t, debug=True)
            gs.append(_check_masks(g, t))
            outs.append(Y)
            dbgs.append(g)
        _check_values(dbgs, outs, np.stack([f64(x) for x in x_gpu]), host, t)
        ref = block.decoder_block(x_ref, host["wqkv"], host["wo"], host["wgu"], host["wd"], host["kc"], host["vc"],
                                  _oracle_t(t))
        flips = 0
        for i in range(8):
            for key, src, tk in (("qkv_in", "xn", "qkv"), ("o_in", "o", "o"), ("gate_up_in", "xn2", "gate_up"),
                                 ("down_in", "h", "down")):
                flips += int((gs[i][key] != teal.magnitude_mask(ref[src][i], t[tk])).sum())
            a, r = gs[i]["down_in"], teal.magnitude_mask(ref["h"][i], t["down"])
            jac.append((a & r).sum() / max(1, (a | r).sum()))
        tot_flips += flips
        x_gpu, x_ref, xc = outs, ref["out"], y_cal
        announce(f"chain block {layer} s={s:.3f} t={[round(v, 5) for v in t.values()]} flips={flips}")
        del host, dev, kcd, vcd, pools
        torch.cuda.empty_cache()
    e2e = max(rel_err(x_gpu[i], x_ref[i]) for i in range(8))
    print(f"32-block chain: mask flips vs fp64 {tot_flips}, down-mask Jaccard min {min(jac):.6f} "
          f"mean {np.mean(jac):.6f}, end-to-end max rel err {e2e:.3e}", flush=True)
    if tot_flips == 0:
        assert e2e < TOL
