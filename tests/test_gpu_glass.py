"""GPU parity of the GLASS static-mask pipeline: local prompt signal (matrix cores),
rank-blend top-k on it, then the neuron-set SwiGLU over decode tokens (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import glass, topk
from helpers import TOL, f64, rel_err, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("P,d,f", [(5, 64, 128), (130, 256, 448), (128, 512, 2048), (1, 128, 64), (17, 384, 192),
                                   (129, 640, 320), (40, 96, 80)])
def test_local_signal_small(P, d, f):
    """Small prompts through both local-signal kernels (d_model a multiple of 128: the
    staged stream, with 1, 2, 3 and 5 stages; otherwise the single-step one), ragged
    token blocks and neuron tiles."""
    announce(f"local signal P={P} d={d} f={f}")
    W = datagen.mlp_weights_neuron_major(4, P, d, f)
    X = datagen.student_t((P, d), 40 + P)
    w = asg.MLPWeights(W.to(DEV), None, L.AS_MLP_NEURON_SET)
    loc = asg.as_glass_local_signal(X.to(DEV), w)
    ref = glass.local_signal(glass.prompt_h(f64(X), f64(W[:, 0]), f64(W[:, 1])))
    assert rel_err(loc, ref) < 1e-5      # fp32 accumulation of exact bf16 products
    assert torch.equal(loc, asg.as_glass_local_signal(X.to(DEV), w))


def test_glass_static_mask_pipeline():
    """d_model 4096, d_ff 14336, bf16: local = mean |h| over a 128-token prompt, prior
    Uniform[0,1), lambda 0.5, keep 7168 neurons, then decode tokens through the
    static-mask SwiGLU."""
    c = datagen.CFG4
    d, f = c["d_model"], c["d_ff"]
    announce("glass pipeline")
    W = datagen.mlp_weights_neuron_major(4, 0, d, f)
    Wd = W.to(DEV)
    w = asg.MLPWeights(Wd, None, L.AS_MLP_NEURON_SET)
    Wg, Wu, Wdn = f64(W[:, 0]), f64(W[:, 1]), f64(W[:, 2])
    prompt = datagen.student_t((c["prompt"], d), datagen.seed_for(4, 0, "prompt"))
    prior = datagen.uniform01((f,), datagen.seed_for(4, 0, "prior"))
    loc = asg.as_glass_local_signal(prompt.to(DEV), w)
    ref_loc = glass.local_signal(glass.prompt_h(f64(prompt), Wg, Wu))
    assert rel_err(loc, ref_loc) < TOL
    # exact index set on the GPU's local scores (stage-wise), and the pure fp64 chain as information
    mask, idx = asg.as_topk_mask(loc, c["keep"], prior=prior.to(DEV), lam=c["lam"])
    ref_idx = topk.glass_topk(f64(loc), f64(prior), c["lam"], c["keep"])
    assert idx.cpu().numpy().tolist() == ref_idx.tolist()
    e2e = topk.glass_topk(ref_loc, f64(prior), c["lam"], c["keep"])
    jac = len(np.intersect1d(e2e, ref_idx)) / len(np.union1d(e2e, ref_idx))
    print(f"jaccard(fp64 chain, GPU chain) = {jac:.6f}", flush=True)
    toks = datagen.student_t((8, d), datagen.seed_for(4, 0, "decode"))
    for i in range(8):
        y = asg.as_sparse_swiglu_mlp(toks[i:i + 1].to(DEV), w, neuron_idx=idx)
        ref = glass.neuron_set_mlp(f64(toks[i:i + 1]), Wg, Wu, Wdn, ref_idx)
        assert rel_err(y, ref) < TOL
