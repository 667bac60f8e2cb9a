"""HIP-graph capture of library calls (the benchmark times sub-steps as graph
replays): every replay must reproduce the eager result bit for bit, with eager
work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        out = fn()
    return g, out


def test_graph_replays_match_eager():
    announce("graph replays")
    shape = datagen.MLPShape(1024, 4096, "bf16")
    wgu, wd = datagen.mlp_weights_input_major(7, 0, shape)
    w = asg.MLPWeights(wgu.to(DEV), wd.to(DEV))
    x = datagen.student_t((1, 1024), 5).to(DEV)
    sc = torch.rand(4096, device=DEV)
    pr = torch.rand(4096, device=DEV)
    eager_y = asg.as_sparse_swiglu_mlp(x, w, 0.7, 0.01).clone()
    eager_k = asg.as_topk_mask(sc, 1000, prior=pr, lam=0.5)[1].clone()
    Y = torch.empty((1, 1024), dtype=torch.float32, device=DEV)

    def step():
        asg.as_sparse_swiglu_mlp(x, w, 0.7, 0.01, Y=Y)
        return asg.as_topk_mask(sc, 1000, prior=pr, lam=0.5)[1]

    g, kout = _capture(step)
    for rep in range(4):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager_y), rep
        assert torch.equal(kout, eager_k), rep
        # eager work between replays
        asg.as_sparse_swiglu_mlp(x, w, 0.3, 0.0)
        torch.cuda.synchronize()


def test_graph_moe_layer_with_side_stream():
    """The MoE layer as captured by the benchmark: the shared expert on a second
    stream, joined by the event the routed experts' down stage waits for; each replay
    equals the eager layer (and the non-overlapped one) bit for bit."""
    announce("graph moe layer")
    w = datagen.moe_weights(5, 3, n_experts=16, d_model=512, d_ff_e=256, d_ff_shared=1024)
    dw = asg.MoEWeights(w["w_gate_up"].to(DEV), w["w_down"].to(DEV), w["w_router"].to(DEV),
                        asg.MLPWeights(w["s_gate_up"].to(DEV), w["s_down"].to(DEV)))
    X = datagen.student_t((2, 512), 12).to(DEV)
    eager = asg.moe_layer(X, dw, 4, 26, one_stream=False).clone()
    serial = asg.moe_layer(X, dw, 4, 26, overlap=False, one_stream=False)
    torch.cuda.synchronize()
    assert torch.equal(eager, serial)
    g, out = _capture(lambda: asg.moe_layer(X, dw, 4, 26, one_stream=False))
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        asg.moe_layer(X, dw, 4, 13, one_stream=False)
        torch.cuda.synchronize()


def test_graph_moe_layer_one_stream():
    """The one-stream MoE layer (as_moe_layer) captured and replayed, with eager calls
    of other keep counts between the replays: every replay equals the eager call."""
    announce("graph moe layer one stream")
    w = datagen.moe_weights(5, 3, n_experts=16, d_model=512, d_ff_e=256, d_ff_shared=1024)
    dw = asg.MoEWeights(w["w_gate_up"].to(DEV), w["w_down"].to(DEV), w["w_router"].to(DEV),
                        asg.MLPWeights(w["s_gate_up"].to(DEV), w["s_down"].to(DEV)))
    X = datagen.student_t((2, 512), 12).to(DEV)
    eager = asg.as_moe_layer(X, dw, 4, 26).clone()
    torch.cuda.synchronize()
    g, out = _capture(lambda: asg.as_moe_layer(X, dw, 4, 26))
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        asg.as_moe_layer(X, dw, 4, 13)
        asg.moe_layer(X, dw, 4, 26, one_stream=False)
        torch.cuda.synchronize()


def test_graph_atomic_splitk_replays():
    """AS_FLAG_ATOMIC_SPLITK under graph replay: the GEMV clears Y with a fill kernel
    (no memset node), the MLP with its gate/up launch, the MoE layer adds onto the
    shared expert's Y; every replay lands within 1e-5 of the eager result (atomic
    additions in any order), with NaN in Y beforehand and eager work in between."""
    announce("graph atomic split-K")
    shape = datagen.MLPShape(1024, 4096, "bf16")
    wgu, wd = datagen.mlp_weights_input_major(7, 0, shape)
    w = asg.MLPWeights(wgu.to(DEV), wd.to(DEV))
    x = datagen.student_t((4, 1024), 6).to(DEV)
    Wg = datagen.normal((4096, 2048), 8).to(DEV)
    xg = datagen.student_t((2, 4096), 9).to(DEV)
    c = datagen.CFG5
    mw = datagen.moe_weights(5, 0, n_experts=c["n_experts"], d_model=c["d_model"], d_ff_e=c["d_ff_e"],
                             d_ff_shared=c["d_ff_shared"])
    dw = asg.MoEWeights(mw["w_gate_up"].to(DEV), mw["w_down"].to(DEV), mw["w_router"].to(DEV),
                        asg.MLPWeights(mw["s_gate_up"].to(DEV), mw["s_down"].to(DEV)))
    xm = datagen.student_t((2, c["d_model"]), 10).to(DEV)
    A = L.AS_FLAG_ATOMIC_SPLITK
    ref_y = asg.as_sparse_swiglu_mlp(x, w, 0.7, 0.01, flags=A).clone()
    ref_g = asg.as_threshold_gemv(xg, Wg, 1.0, flags=A).clone()
    ref_m = asg.moe_layer(xm, dw, c["top"], c["keep"], flags=A).clone()
    Y = torch.empty((4, 1024), dtype=torch.float32, device=DEV)
    G = torch.empty((2, 2048), dtype=torch.float32, device=DEV)

    def step():
        asg.as_sparse_swiglu_mlp(x, w, 0.7, 0.01, flags=A, Y=Y)
        asg.as_threshold_gemv(xg, Wg, 1.0, flags=A, Y=G)
        return asg.moe_layer(xm, dw, c["top"], c["keep"], flags=A)

    g, mout = _capture(step)

    def close(a, b):
        return float((a - b).abs().max()) <= 1e-5 * float(b.abs().max())

    for rep in range(4):
        Y.fill_(float("nan"))
        G.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert close(Y, ref_y), rep
        assert close(G, ref_g), rep
        assert close(mout, ref_m), rep
        asg.as_sparse_swiglu_mlp(x, w, 0.3, 0.0)
        torch.cuda.synchronize()
