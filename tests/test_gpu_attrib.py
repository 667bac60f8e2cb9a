"""GPU parity of attribution-based selection: Corrected GxO scores, per-layer top
fraction, and the head-masked output projection (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import attrib, glass
from helpers import f64, rel_err, bits_to_bool, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("rows,n", [(1, 100), (4, 14336), (32, 4096), (3, 257)])
def test_corrected_gxo(rows, n):
    announce(f"corrected gxo {rows}x{n}")
    x = datagen.student_t((rows, n), 70 + n, dtype="f32")
    g = datagen.normal((rows, n), 80 + n, std=1e-3, dtype="f32")
    s = asg.as_corrected_gxo(x.to(DEV), g.to(DEV))
    assert rel_err(s, attrib.corrected_gxo(f64(x), f64(g))) < 2e-6
    assert torch.equal(s, asg.as_corrected_gxo(x.to(DEV), g.to(DEV)))


@pytest.mark.parametrize("num,den", [(3, 10), (2, 5), (1, 1), (0, 1), (1, 3)])
def test_top_fraction_exact_on_gpu_scores(num, den):
    """The kept set of every layer equals the oracle's top fraction of the GPU's own
    scores, bit for bit (ties from rounded scores, a NaN, negative scores)."""
    rows, n = 32, 4096
    x = datagen.student_t((rows, n), 5, dtype="f32")
    g = datagen.normal((rows, n), 6, std=1e-3, dtype="f32")
    s = asg.as_corrected_gxo(x.to(DEV), g.to(DEV))
    s = torch.round(s * 64) / 64                    # ties
    s[3, 17] = float("nan")
    mask, idx = asg.as_select_top_fraction(s, num, den)
    keep = attrib.top_fraction(f64(s), num, den)
    assert np.array_equal(bits_to_bool(mask, n), keep)
    k = attrib.fraction_count(n, num, den)
    assert idx.shape == (rows, k)
    for r in range(rows):
        assert idx[r].cpu().numpy().tolist() == np.flatnonzero(keep[r]).tolist()


def test_top_fraction_feeds_the_neuron_set_mlp():
    """External scores -> the top 40% of d_ff 14336 neurons -> the neuron-set SwiGLU;
    the output matches the fp64 neuron-set MLP on the same kept set."""
    d, f = 4096, 14336
    W = datagen.mlp_weights_neuron_major(9, 0, d, f)
    w = asg.MLPWeights(W.to(DEV), None, L.AS_MLP_NEURON_SET)
    score = datagen.normal((1, f), 11, std=1.0, dtype="f32").to(DEV)
    _, idx = asg.as_select_top_fraction(score, 2, 5)
    tok = datagen.student_t((1, d), 12)
    y = asg.as_sparse_swiglu_mlp(tok.to(DEV), w, neuron_idx=idx[0].contiguous())
    I = idx[0].cpu().numpy()
    ref = glass.neuron_set_mlp(f64(tok), f64(W[:, 0]), f64(W[:, 1]), f64(W[:, 2]), I)
    assert len(I) == 5735
    assert rel_err(y, ref) < 2e-5


@pytest.mark.parametrize("nh,hd,N,keep", [(32, 128, 4096, [0, 5, 9, 31]), (32, 128, 4096, list(range(0, 32, 2))),
                                          (8, 64, 1024, []), (12, 96, 768, list(range(12)))])
def test_head_masked_gemv(nh, hd, N, keep):
    announce(f"head gemv nh={nh} hd={hd} N={N} keep={len(keep)}")
    x = datagen.student_t((nh * hd,), 30 + N)
    W = datagen.normal((nh * hd, N), 40 + N)
    heads = torch.tensor(keep if keep else [0], dtype=torch.int32, device=DEV)[:len(keep)]
    y = asg.as_head_masked_gemv(x.to(DEV), W.to(DEV), heads, nh, hd)
    ref = attrib.head_masked_gemv(f64(x), f64(W), keep, hd)
    if keep:
        assert rel_err(y, ref) < 2e-5
    else:
        assert torch.count_nonzero(y).item() == 0


def test_head_masked_gemv_integer_exact():
    nh, hd, N = 32, 128, 4096
    x = datagen.int_valued((nh * hd,), 7, -4, 4)
    W = datagen.int_valued((nh * hd, N), 8, -3, 3)
    keep = [1, 2, 3, 17, 30]
    heads = torch.tensor(keep, dtype=torch.int32, device=DEV)
    y = asg.as_head_masked_gemv(x.to(DEV), W.to(DEV), heads, nh, hd)
    assert np.array_equal(f64(y), attrib.head_masked_gemv(f64(x), f64(W), keep, hd))
